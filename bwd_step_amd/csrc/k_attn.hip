// Causal softmax attention, forward and backward ("nanochat explainer",
// The Full Pipeline -> Pretraining: causal next-token prediction; Inference &
// KV Cache: full multi-head attention; One Dial: head_dim 128).
//
//   o_t = sum_{j<=t} P_tj v_j,  P_tj = exp(s_tj - lse_t),  s_tj = qh_t . kh_j / sqrt(hd)
//   backward: D_t = do_t . o_t; dv_j = sum_t P_tj do_t; dS = P (do v^T - D);
//             dqh_t = sum_j dS_tj kh_j / sqrt(hd); dkh_j = sum_t dS_tj qh_t / sqrt(hd)
//
// bf16 path (MFMA, v_mfma_f32_32x32x16_bf16, fp32 accumulation), head_dim 64
// or 128.  Every wavefront keeps its 32 queries (or keys) in the MFMA column
// dimension, so each lane owns one query: the softmax statistics and the
// output rescale are lane-local and only the row maximum needs one exchange
// with the partner lane (lane ^ 32).  Scores are computed transposed
// (S^T = K Q^T, A operand from an LDS K tile, B operand = Q held in
// registers) and the output as O^T = V^T P^T, whose B operand is exactly the
// score accumulator converted to bf16; V^T comes from the row-major V tile
// through transposed LDS reads (head_dim 128) or from a tile transposed in
// registers while it is staged (head_dim 64).  The key order inside one MFMA
// reduction step is permuted identically in both operands, which leaves the
// sum unchanged.
//
// Forward: 128 queries per workgroup (4 wavefronts x 32), 64-key blocks,
// online softmax in the exp2 domain; lse is saved.  Backward, head_dim 128:
// D = rowsum(dO * O), then a dK/dV kernel (128 keys per workgroup, two
// wavefronts per 32 keys, looping over 64-query blocks with P recomputed
// from lse) that also stores -dS and finishes the QK-norm + RoPE backward of
// k, then a dQ kernel from the stored dS (two 256-query tiles per workgroup)
// that finishes that of q; head_dim 64: dK/dV and dQ kernels that each
// recompute P (128 keys or queries per workgroup).  No floating-point
// atomics, so results are reproducible.  Workgroups with the most causal
// work are launched first.
//
// fp32 debug path: one wavefront per query (forward, dQ) or per key (dK/dV),
// plain loops over the causal range.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace nc {

constexpr float kLog2e = 1.4426950408889634f;

// 2^x with the hardware instruction (no range fix-up; results below the
// smallest normal flush to zero, which is harmless for softmax weights).
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Tile staging: a [64 rows][HD] bf16 tile is read in 4-row x 8-column blocks
// (four 16-byte loads).  The same registers can be stored row-major
// (row stride HD + 8) and/or transposed (row stride 64 + 4).
template <int HD>
struct KvStage {
  static constexpr int BLOCKS = (64 / 4) * (HD / 8);  // 4x8 blocks per tile
  u32x4 r[4];
  bool active;
  int row0, col0;

  __device__ __forceinline__ void load(const bf16* __restrict__ base, long ld, int t0, int T) {
    const int blk = threadIdx.x;
    active = blk < BLOCKS;
    row0 = (blk / (HD / 8)) * 4;
    col0 = (blk % (HD / 8)) * 8;
    if (!active) return;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int t = t0 + row0 + q;
      if (t < T)
        r[q] = *reinterpret_cast<const u32x4*>(base + (size_t)t * ld + col0);
      else
        r[q] = u32x4{0, 0, 0, 0};
    }
  }
  __device__ __forceinline__ void store_rows(bf16* __restrict__ s) const {
    if (!active) return;
#pragma unroll
    for (int q = 0; q < 4; ++q) *reinterpret_cast<u32x4*>(s + (row0 + q) * (HD + 8) + col0) = r[q];
  }
  __device__ __forceinline__ void store_cols(bf16* __restrict__ s) const {
    if (!active) return;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
      const int w = c >> 1;
      u32x2 o;
      o.x = __builtin_amdgcn_perm(r[1][w], r[0][w], sel);
      o.y = __builtin_amdgcn_perm(r[3][w], r[2][w], sel);
      *reinterpret_cast<u32x2*>(s + (col0 + c) * (64 + 4) + row0) = o;
    }
  }
};

// Two 8-byte reads (4 bf16 each) from a transposed tile: elements
// [row][c0 .. c0+3] and [row][c0+8 .. c0+11].
__device__ __forceinline__ bf16x8 read_t8(const bf16* s, int row, int c0) {
  const u32x2 lo = *reinterpret_cast<const u32x2*>(s + row * (64 + 4) + c0);
  const u32x2 hi = *reinterpret_cast<const u32x2*>(s + row * (64 + 4) + c0 + 8);
  u32x4 v{lo.x, lo.y, hi.x, hi.y};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x8 pack8(const f32x16& a, int t) {
  u32x4 v;
  v.x = pack_bf16x2(a[t * 8 + 0], a[t * 8 + 1]);
  v.y = pack_bf16x2(a[t * 8 + 2], a[t * 8 + 3]);
  v.z = pack_bf16x2(a[t * 8 + 4], a[t * 8 + 5]);
  v.w = pack_bf16x2(a[t * 8 + 6], a[t * 8 + 7]);
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row (in the MFMA M dimension) held by accumulator register r of a lane in
// half `g` (= lane / 32) of the wavefront.
__device__ __forceinline__ int acc_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

// Workgroup order for the attention kernels: workgroups are dealt to the 8
// XCDs round-robin, so consecutive logical blocks (the key or query blocks of
// one (batch, head)) are remapped onto one XCD, where they share Q/dO or K/V
// in its L2.
__device__ __forceinline__ int xcd_block(int lin, int n) {
  return (n & 7) == 0 ? (lin & 7) * (n >> 3) + (lin >> 3) : lin;
}

// ------------------------------------------------------------------ forward
template <int HD>
__global__ void __launch_bounds__(256) attn_fwd_mfma(AttnArgs p) {
  constexpr int KS = HD / 16, HB = HD / 32;
  __shared__ __attribute__((aligned(16))) bf16 Ks[64 * (HD + 8)];
  __shared__ __attribute__((aligned(16))) bf16 Vt[HD * (64 + 4)];

  const int T = p.T;
  const int nqb = gridDim.x;  // (T + 127) / 128
  const int lin = xcd_block(blockIdx.x + nqb * blockIdx.y, nqb * gridDim.y);
  const int qb = nqb - 1 - lin % nqb;  // query blocks of one (b, h) in turn on one XCD, the longest first
  const int bh = lin / nqb, b = bh / p.H, h = bh % p.H;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 5, li = lane & 31;
  const int q0 = qb * 128;
  const int qi = q0 + wv * 32 + li;
  const size_t tok0 = (size_t)b * T;

  const bf16* qp = (const bf16*)p.q + tok0 * p.ldq + h * HD;
  const bf16* kp = (const bf16*)p.k + tok0 * p.ldk + (h / p.G) * HD;
  const bf16* vp = (const bf16*)p.v + tok0 * p.ldv + (h / p.G) * HD;

  bf16x8 qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s)
    qf[s] = qi < T ? *reinterpret_cast<const bf16x8*>(qp + (size_t)qi * p.ldq + s * 16 + g * 8) : bf16x8{};

  f32x16 oacc[HB];
#pragma unroll
  for (int x = 0; x < HB; ++x) oacc[x] = f32x16{};
  float mx = -INFINITY, lsum = 0.f;

  const int q_last = min(T - 1, q0 + 127);
  const int nkv = q_last / 64 + 1;
  const int wq_min = q0 + wv * 32, wq_max = wq_min + 31;

  KvStage<HD> sk, sv;
  sk.load(kp, p.ldk, 0, T);
  sv.load(vp, p.ldv, 0, T);
  for (int kb = 0; kb < nkv; ++kb) {
    __syncthreads();
    sk.store_rows(Ks);
    sv.store_cols(Vt);
    __syncthreads();
    if (kb + 1 < nkv) {
      sk.load(kp, p.ldk, (kb + 1) * 64, T);
      sv.load(vp, p.ldv, (kb + 1) * 64, T);
    }
    const int kbase = kb * 64;
    if (kbase > wq_max) continue;  // every key of this block is in this wave's future

    f32x16 sacc[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      sacc[kk] = f32x16{};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Ks + (kk * 32 + li) * (HD + 8) + s * 16 + g * 8);
        sacc[kk] = mfma(kf, qf[s], sacc[kk]);
      }
    }
    const bool need_mask = (kbase + 63 > wq_min) || (kbase + 64 > T);
    float lmax = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = sacc[kk][r] * p.scale_log2;
        if (need_mask) {
          const int key = kbase + kk * 32 + acc_row(r, g);
          if (key > qi || key >= T) v = -INFINITY;
        }
        sacc[kk][r] = v;
        lmax = fmaxf(lmax, v);
      }
    lmax = fmaxf(lmax, __shfl_xor(lmax, 32, 64));
    const float mnew = fmaxf(mx, lmax);
    const float alpha = exp2f(mx - mnew);
    float ps = 0.f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = exp2f(sacc[kk][r] - mnew);
        sacc[kk][r] = e;
        ps += e;
      }
    lsum = lsum * alpha + ps;
    mx = mnew;
#pragma unroll
    for (int x = 0; x < HB; ++x) oacc[x] *= alpha;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8 pf = pack8(sacc[kk], t);
#pragma unroll
        for (int x = 0; x < HB; ++x) {
          const bf16x8 vf = read_t8(Vt, x * 32 + li, kk * 32 + t * 16 + 4 * g);
          oacc[x] = mfma(vf, pf, oacc[x]);
        }
      }
  }
  const float ltot = lsum + __shfl_xor(lsum, 32, 64);
  if (qi >= T) return;
  const float inv = 1.0f / ltot;
  bf16* op = (bf16*)p.o + (tok0 + qi) * p.ldo + h * HD;
#pragma unroll
  for (int x = 0; x < HB; ++x)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      u32x2 w;
      w.x = pack_bf16x2(oacc[x][rg * 4 + 0] * inv, oacc[x][rg * 4 + 1] * inv);
      w.y = pack_bf16x2(oacc[x][rg * 4 + 2] * inv, oacc[x][rg * 4 + 3] * inv);
      *reinterpret_cast<u32x2*>(op + x * 32 + 8 * rg + 4 * g) = w;
    }
  if (g == 0) p.lse[(size_t)bh * T + qi] = mx + log2f(ltot);  // base 2
}

// ------------------------------------------------------------------ head_dim 128 helpers
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#define LDS_AS __attribute__((address_space(3)))
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// chunk swizzle of the forward's V tile: key & 3 -> XOR of the 16-byte chunk
// index, so that the transposed reads of four consecutive keys are conflict free
__device__ __forceinline__ int sw_v(int r) { return 4 * r + 2 * ((r >> 1) & 1); }
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ------------------------------------------------------------------ backward, head_dim 128
// Tiles of 64 rows x 128 that are read both ways -- 16-byte row fragments
// (the A operand of S = Q K^T, dP = dO V^T and their transposes) and
// transposed fragments through ds_read_b64_tr_b16 (the A operand of
// dQ^T = K^T dS^T, dK^T = Q^T dS, dV^T = dO^T P) -- use one XOR swizzle of
// the 16-byte chunk index, sw2(row), that is conflict free for both access
// patterns (any 16 aligned rows see 16 distinct chunk slots; within every
// aligned group of 4 rows bits 2-3 differ and bits 1-2 differ).
__device__ __forceinline__ int sw2(int row) { return 4 * (row & 3) + (((row >> 2) & 3) ^ (2 * ((row >> 1) & 1))); }

// Transposed fragment: A-operand rows = columns x*32 + (lane & 31) of the
// tile, reduction index = tile rows kb + {4g .. 4g+3, 8+4g .. 8+4g+3}.
__device__ __forceinline__ bf16x8 tr_frag(const bf16* S, int x, int kb, int lane) {
  const int gi = lane >> 4, i = lane & 15;
  const int r = i >> 2, q = i & 3;
  const int chunk = x * 4 + 2 * (gi & 1) + (q >> 1);
  const int k0 = kb + 4 * (gi >> 1) + r;
  const int sub = 4 * (q & 1);
  const v4i16 lo =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)(S + k0 * 128 + ((chunk ^ sw2(k0)) << 3) + sub));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (LDS_AS v4i16*)(S + (k0 + 8) * 128 + ((chunk ^ sw2(k0 + 8)) << 3) + sub));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// LDS-direct load written as inline assembly: 64 lanes x 16 bytes from the
// buffer into the 1-KB LDS slot at byte address `lds`.  The compiler does not
// see these loads, so it adds no waits of its own for them: the kernels
// that use this count them and wait explicitly (s_waitcnt vmcnt), and the
// barrier asm that follows carries a memory clobber, so no LDS read moves
// above it.  m0 (the LDS destination) is saved and restored.
__device__ __forceinline__ void dma16(rsrc_t rs, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(rs)
      : "memory");
}

// The same load with the non-temporal policy (data read once, streamed).
__device__ __forceinline__ void dma16_nt(rsrc_t rs, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen nt lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(rs)
      : "memory");
}

// The stored dS of one (b, h), lane-major.  The dK/dV kernel holds -dS^T
// of 32 keys (a key block kw) x 32 queries (a query block qw) in one
// wavefront as two B-operand fragments per lane: fragment t of lane
// l = li + 32 g holds key 32 kw + li and queries 32 qw + 16 t + 4 g + {0..3},
// 32 qw + 16 t + 8 + 4 g + {0..3}.  Each fragment is stored whole, so chunk
// (kw, qw, t) is 1 KB with lane l's 16 bytes at byte 16 l, and a store
// instruction writes one contiguous KB.  Chunks are ordered kw, qw, t; a
// (b, h) takes (Tp / 32)^2 * 2 KB = Tp^2 * 2 bytes.
__device__ __forceinline__ uint32_t ds_chunk(long Tp, int kw, int qw, int t) {
  return (uint32_t)((((long)kw * (Tp >> 5) + qw) * 2 + t) * 1024);
}

// ------------------------------------------------------------------ forward, head_dim 128
// Forward, head_dim 128: 128 queries per workgroup (4 wavefronts x 32, Q
// fragments in registers), 64-key blocks of K and V through two LDS stages
// (one array: K of stage 0 and 1, then V of stage 0 and 1, 16 KB each)
// loaded one block ahead by inline-asm LDS-direct loads (a key past T reads
// 0 through the buffer range check).  S^T = K Q^T with K fragments as 16-byte
// reads of the row tile (chunk ^= key & 15); O^T = V^T P^T with V^T
// fragments through ds_read_b64_tr_b16 from the row tile (chunks swizzled by
// sw_v(key & 3)); both read without bank conflicts.  Every fragment address
// is a per-lane register (moved to the block's stage once per block) plus an
// immediate.  The row sum
// of P is taken from the bf16 values that enter the product (v_dot2 with
// ones), so the normalisation matches the numerator.  The kernel stays under
// 256 registers per lane so that two workgroups (eight wavefronts) share a
// compute unit and one's softmax overlaps the other's MFMAs.
__global__ void __launch_bounds__(256, 2) attn_fwd128(AttnArgs p) {
  constexpr int HD = 128, KS = 8, HB = 4;
  constexpr uint32_t kTile = 64 * HD * 2, kVs = 2 * kTile;
  __shared__ __attribute__((aligned(1024))) char smem[4 * kTile];
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  const int T = p.T;
  const int nqb = gridDim.x;  // (T + 127) / 128
  const int lin = xcd_block(blockIdx.x + nqb * blockIdx.y, nqb * gridDim.y);
  const int qb = nqb - 1 - lin % nqb;  // query blocks of one (b, h) in turn on one XCD, the longest first
  const int bh = lin / nqb, b = bh / p.H, h = bh % p.H;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, li = lane & 31;
  const int q0 = qb * 128;
  const int qi = q0 + wv * 32 + li;
  const size_t tok0 = (size_t)b * T;
  const uint32_t kbytes = (uint32_t)(((size_t)(T - 1) * p.ldk + (size_t)(p.H / p.G) * HD) * 2);
  const uint32_t vbytes = (uint32_t)(((size_t)(T - 1) * p.ldv + (size_t)(p.H / p.G) * HD) * 2);
  const rsrc_t rk = make_rsrc((const bf16*)p.k + tok0 * p.ldk, kbytes);
  const rsrc_t rv = make_rsrc((const bf16*)p.v + tok0 * p.ldv, vbytes);
  const long colk = (long)(h / p.G) * HD;  // this query head's key/value head

  const bf16* qp = (const bf16*)p.q + tok0 * p.ldq + h * HD;
  bf16x8 qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s)
    qf[s] = qi < T ? *reinterpret_cast<const bf16x8*>(qp + (size_t)qi * p.ldq + s * 16 + g * 8) : bf16x8{};
  // wait for Q here: the compiler does not see the asm loads' waits and
  // would otherwise wait for every load at the first use of Q in the loop
#pragma unroll
  for (int s = 0; s < KS; ++s) asm volatile("" ::"v"(qf[s]));

  // this wavefront's loads of a block: 1-KB slots wv * 4 + i (key rows
  // 4 slot .. + 3) of the K and V tiles; per-lane byte offsets relative to
  // the block's first key.  A row at or past T lies past the buffer's range
  // (the last row ends at the last head's column), so it reads 0.
  uint32_t ko[4], vo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (wv * 4 + i) * 4 + (lane >> 4);
    const int pc = lane & 15;
    ko[i] = (uint32_t)(((long)row * p.ldk + colk + ((pc ^ (row & 15)) << 3)) * 2);
    vo[i] = (uint32_t)(((long)row * p.ldv + colk + ((pc ^ sw_v(row & 3)) << 3)) * 2);
  }
  auto load_kv = [&](uint32_t st, int key0) __attribute__((always_inline)) {
    const uint32_t rk0 = (uint32_t)key0 * (uint32_t)p.ldk * 2u, rv0 = (uint32_t)key0 * (uint32_t)p.ldv * 2u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t slot = st * kTile + (uint32_t)(wv * 4 + i) * 1024u;
      dma16(rk, ko[i] + rk0, lds0 + slot);
      dma16(rv, vo[i] + rv0, lds0 + kVs + slot);
    }
  };

  // Per-lane LDS byte offsets of the fragment reads, formed once (opaque to
  // the compiler so that it neither re-derives them nor hoists sums with the
  // immediates): K fragment s of key row li (+8 KB for keys 32..63 of the
  // block), V^T fragment x (keys 4 (gi >> 1) + r; +2 KB for the other eight
  // of the 16-key step, +4 KB per step).
  uint32_t kfo[KS], vfo[HB];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    kfo[s] = (uint32_t)(li * 256 + (((2 * s + g) ^ (li & 15)) << 4));
    asm volatile("" : "+v"(kfo[s]));
  }
  {
    const int gi = lane >> 4, i = lane & 15, r = i >> 2, q = i & 3;
#pragma unroll
    for (int x = 0; x < HB; ++x) {
      const int chunk = (x * 4 + 2 * (gi & 1) + (q >> 1)) ^ sw_v(r);
      vfo[x] = kVs + (uint32_t)((4 * (gi >> 1) + r) * 256 + chunk * 16 + 8 * (q & 1));
      asm volatile("" : "+v"(vfo[x]));
    }
  }
  auto kfrag = [&](uint32_t imm, int s) { return *reinterpret_cast<const bf16x8*>(smem + imm + kfo[s]); };
  auto vtfrag = [&](uint32_t imm, int x) {
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)(smem + imm + vfo[x]));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)(smem + imm + 2048u + vfo[x]));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x16 oacc[HB];
#pragma unroll
  for (int x = 0; x < HB; ++x) oacc[x] = f32x16{};
  float mx = -INFINITY, lsum = 0.f;
  const float c = p.scale_log2;
  const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);

  const int q_last = min(T - 1, q0 + 127);
  const int nkv = q_last / 64 + 1;
  const int wq_min = q0 + wv * 32, wq_max = wq_min + 31;

  load_kv(0, 0);
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");

  // key block kb in stage kb & 1; the loads of block kb + 1 (or, past the
  // last, of rows past T) go to the other stage.  The fragment offsets move
  // to the block's stage by a uniform delta.
  auto block = [&](int kb) __attribute__((always_inline)) {
    const uint32_t st = (uint32_t)kb & 1u;
    if (kb > 0) {
      const uint32_t d = st ? kTile : (uint32_t)-(int)kTile;
#pragma unroll
      for (int s = 0; s < KS; ++s) kfo[s] += d;
#pragma unroll
      for (int x = 0; x < HB; ++x) vfo[x] += d;
      asm volatile("" : "+v"(kfo[0]), "+v"(kfo[1]), "+v"(kfo[2]), "+v"(kfo[3]), "+v"(kfo[4]), "+v"(kfo[5]),
                   "+v"(kfo[6]), "+v"(kfo[7]), "+v"(vfo[0]), "+v"(vfo[1]), "+v"(vfo[2]), "+v"(vfo[3]));
    }
    load_kv(st ^ 1u, kb + 1 < nkv ? (kb + 1) * 64 : T);
    const int kbase = kb * 64;
    if (kbase <= wq_max) {
      f32x16 sacc[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        sacc[kk] = f32x16{};
#pragma unroll
        for (int s = 0; s < KS; ++s) sacc[kk] = mfma(kfrag(kk * 8192u, s), qf[s], sacc[kk]);
      }
      const bool need_mask = (kbase + 63 > wq_min) || (kbase + 64 > T);
      float lmax = -INFINITY;
      if (need_mask) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kbase + kk * 32 + acc_row(r, g);
            if (key > qi || key >= T) sacc[kk][r] = -INFINITY;
          }
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int r = 0; r < 16; ++r) lmax = fmaxf(lmax, sacc[kk][r]);
      lmax = fmaxf(lmax, __shfl_xor(lmax, 32, 64));
      // Running max in the scaled log2 domain.  It is raised (and O and the
      // sum rescaled) only when a score exceeds it by more than 8, so the
      // weights below stay <= 2^8 and the costly rescale is rare; the final
      // normalisation by the sum makes the result independent of the choice.
      const float mcand = fmaxf(mx, lmax * c);
      if (mcand > mx + 8.f) {
        const float alpha = ex2(mx - mcand);
        lsum *= alpha;
#pragma unroll
        for (int x = 0; x < HB; ++x) oacc[x] *= alpha;
        mx = mcand;
      }
      const float moff = mx == -INFINITY ? 0.f : -mx;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kk][r] = ex2(fmaf(sacc[kk][r], c, moff));
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const bf16x8 pf = pack8(sacc[kk], t);
          // (the pairs are taken with shufflevector: a bit_cast of a 32-bit
          // lane to bf16x2 here selects the wrong register on this compiler)
          lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 0, 1), ones, lsum, false);
          lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 2, 3), ones, lsum, false);
          lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 4, 5), ones, lsum, false);
          lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 6, 7), ones, lsum, false);
#pragma unroll
          for (int x = 0; x < HB; ++x)
            oacc[x] = mfma(vtfrag((uint32_t)(kk * 32 + t * 16) * 256u, x), pf, oacc[x]);
        }
    }
    // this wavefront's loads of block kb + 1 landed and every wavefront is
    // done reading this block's stage
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };

  for (int kb = 0; kb < nkv; ++kb) block(kb);

  const float ltot = lsum + __shfl_xor(lsum, 32, 64);
  if (qi >= T) return;
  const float inv = 1.0f / ltot;
  bf16* op = (bf16*)p.o + (tok0 + qi) * p.ldo + h * HD;
#pragma unroll
  for (int x = 0; x < HB; ++x)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      u32x2 w;
      w.x = pack_bf16x2(oacc[x][rg * 4 + 0] * inv, oacc[x][rg * 4 + 1] * inv);
      w.y = pack_bf16x2(oacc[x][rg * 4 + 2] * inv, oacc[x][rg * 4 + 3] * inv);
      *reinterpret_cast<u32x2*>(op + x * 32 + 8 * rg + 4 * g) = w;
    }
  if (g == 0) p.lse[(size_t)bh * T + qi] = mx + log2f(ltot);  // base 2
}

// D = rowsum(dO * O) of every (token, head), head_dim 128: 16 lanes per row
// (16 bytes of each operand per lane, so four whole rows per wavefront
// load), reduced across the 16 lanes; stored [b * H + h][t] for the dK/dV
// kernel.
__global__ void __launch_bounds__(256) attn_bwd_D128(AttnArgs p) {
  const long row = (long)blockIdx.x * 16 + (threadIdx.x >> 4);  // (b T + t) H + h
  const int l = threadIdx.x & 15;
  const long rows = (long)p.B * p.T * p.H;
  const long n = row / p.H;
  const int h = (int)(row - n * p.H);
  float s = 0.f;
  if (row < rows) {
    const u32x4 a = *reinterpret_cast<const u32x4*>((const bf16*)p.o + n * p.ldo + h * 128 + l * 8);
    const u32x4 b = *reinterpret_cast<const u32x4*>((const bf16*)p.dout + n * p.lddo + h * 128 + l * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      s = fmaf(bf16lo_to_f32(a[w]), bf16lo_to_f32(b[w]), s);
      s = fmaf(bf16hi_to_f32(a[w]), bf16hi_to_f32(b[w]), s);
    }
  }
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) s += __shfl_xor(s, o, 16);
  if (row < rows && l == 0) {
    const long b = n / p.T, t = n - b * p.T;
    p.Dbuf[((size_t)b * p.H + h) * p.T + t] = s;
  }
}

// dQ from the stored dS: dQ_t = scale sum_j dS_tj kh_j, as dQ^T = K^T dS^T.
// The A operand is transposed out of the K tile (tr_frag); the B operand
// comes from the dS chunks with ds_read_b64_tr_b16 (ds_frag).  The dK/dV
// kernel stored every chunk of its 128 keys from their first query on
// (zeros above the diagonal and past T), so no mask is needed; a wavefront
// only skips the key blocks past its last query.  Tiles of 256 queries (8
// wavefronts of 32, two per SIMD), 64-key blocks through three LDS stages (a
// K tile, 64 rows x 256 bytes with the sw2 swizzle, and the 32 dS chunks of
// 64 keys x 256 queries; 48 KB each), loaded two blocks ahead.  A workgroup
// runs two tiles of one (b, h), i and n - 1 - i, so all workgroups have equal
// work and those of one (b, h) read the same K blocks together from their
// XCD's L2; the stored dS, read once, is loaded with the non-temporal
// policy.  The epilogue of each tile also runs the QK-norm + RoPE backward
// of q, so it writes the gradient w.r.t. the pre-norm q.
//
// In LDS the chunks are ordered (kw, qw, t) within the tile and the 16-byte
// piece of chunk lane li + 32 g sits at slot 32 g + (li ^ (4 g + 8 t)): the
// 32 lanes of each half of a transposed read then cover 64 distinct banks.
template <int QW>  // 32-query blocks of the tile (chunks per 32 keys: 2 QW)
__device__ __forceinline__ bf16x8 ds_frag(const bf16* S, int qwl, int kb, int lane) {
  const int gi = lane >> 4, i = lane & 15;
  const int r = i >> 2, q = i & 3;
  const int gq = q & 1;  // the fragment half (g of the storing lane) that holds queries 4q .. 4q+3
  const int k0 = kb + 4 * (gi >> 1) + r;
  const int t = gi & 1;  // the 16-query half: chunk parity
  auto addr = [&](int kk) {
    const int chunk = (kk >> 5) * (2 * QW) + qwl * 2 + t;
    const int slot = 32 * gq + ((kk & 31) ^ (4 * gq + 8 * t));
    return (LDS_AS v4i16*)(S + chunk * 512 + slot * 8 + 4 * (q >> 1));
  };
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(addr(k0));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(addr(k0 + 8));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

constexpr int kDqQueries = 256;  // queries per workgroup of the dQ kernel
constexpr bool kDqDsNt = true;    // stored dS read with the non-temporal policy

__global__ void __launch_bounds__(512, 1) attn_bwd_dq_ds128(AttnArgs p) {
  constexpr int HD = 128, HB = 4, QW = kDqQueries / 32;
  constexpr uint32_t kTile = 64 * HD * 2, kStage = kTile + 64 * kDqQueries * 2;
  __shared__ __attribute__((aligned(1024))) char smem[3 * kStage];
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  const int T = p.T;
  const long Tp = p.tpad;
  // Workgroup pi of a (b, h) takes query tiles ntile - 1 - pi and pi (the
  // longer first), so every workgroup has the same number of key blocks and
  // the workgroups of one (b, h), started together on one XCD, walk the same
  // K blocks at the same time (shared in its L2).
  const int ntile = (T + kDqQueries - 1) / kDqQueries;
  const int npg = gridDim.x;  // (ntile + 1) / 2
  const int lin = xcd_block(blockIdx.x + npg * blockIdx.y, npg * gridDim.y);
  const int pi = lin % npg;
  const int bh = lin / npg, b = bh / p.H, h = bh % p.H;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5;
  const size_t tok0 = (size_t)b * T;
  const rsrc_t rk = make_rsrc((const bf16*)p.k + tok0 * p.ldk,
                              (uint32_t)(((size_t)(T - 1) * p.ldk + (size_t)(p.H / p.G) * HD) * 2));
  const rsrc_t rs = make_rsrc((const bf16*)p.dsT + (size_t)bh * Tp * Tp, (uint32_t)(Tp * Tp * 2));
  const long col = (long)(h / p.G) * HD;  // this query head's key/value head

  // K tile: per-lane byte offsets of this wavefront's 2 blocks (4 rows each)
  // relative to the key block's first row.  dS: this wavefront loads chunks
  // 4 wv .. 4 wv + 3 of the tile; LDS slot `lane` of a chunk of parity t
  // takes the stored piece of lane (li ^ (4 g + 8 t)) + 32 g.
  uint32_t toff_k[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = (wv * 2 + i) * 4 + (lane >> 4);
    const int cc = (lane & 15) ^ sw2(row);
    toff_k[i] = (uint32_t)(((long)row * p.ldk + col + cc * 8) * 2);
  }
  const uint32_t src_lane[2] = {(uint32_t)((((lane & 31) ^ (4 * g)) + 32 * g) * 16),
                                 (uint32_t)((((lane & 31) ^ (4 * g + 8)) + 32 * g) * 16)};
  for (int pass = 0; pass < 2; ++pass) {
    const int qb = pass == 0 ? ntile - 1 - pi : pi;
    if (pass == 1) {
      if (qb == ntile - 1 - pi) break;  // the middle tile of an odd count runs once
      // every wavefront is done with the last stage of the first tile
      __syncthreads();
    }
    const int q0 = qb * kDqQueries;
    const int qi = q0 + wv * 32 + (lane & 31);  // this lane's query
    const int nkv = min(T - 1, q0 + kDqQueries - 1) / 64 + 1;  // key blocks up to the diagonal
    // the loads of key block j into stage st; blocks past the last read 0
    auto load_block = [&](int st, int j) {
      const bool live = j < nkv;
      const int row0 = j * 64;
      const uint32_t sb = lds0 + (uint32_t)st * kStage;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const bool ok = live && row0 + (wv * 2 + i) * 4 + (lane >> 4) < T;  // keys past T read 0
        dma16(rk, ok ? toff_k[i] + (uint32_t)(row0 * p.ldk * 2) : kOOB, sb + (uint32_t)(wv * 2 + i) * 1024u);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // chunk (kwl, qwl, t) = (c / (2 QW), (c / 2) % QW, c % 2); c % 2 = i % 2.  A
        // query block past the padded length reads 0 (its queries are past T).
        const int c = wv * 4 + i;
        const int qw = (q0 >> 5) + ((c >> 1) % QW);
        const uint32_t off = live && qw < (int)(Tp >> 5) ? src_lane[i & 1] + ds_chunk(Tp, 2 * j + c / (2 * QW), qw, c & 1) : kOOB;
        if constexpr (kDqDsNt) dma16_nt(rs, off, sb + kTile + (uint32_t)c * 1024u);
        else dma16(rs, off, sb + kTile + (uint32_t)c * 1024u);
      }
    };

    f32x16 dq[HB];
#pragma unroll
    for (int x = 0; x < HB; ++x) dq[x] = f32x16{};

    load_block(0, 0);
    load_block(1, 1);
    int cur = 0;  // stage of block j
    for (int j = 0; j < nkv; ++j) {
      // loads retire in issue order: with those of block j + 1 (6) still in
      // flight, block j has landed; after the barrier every wavefront is done
      // with block j - 1, whose stage the loads of block j + 2 take
      asm volatile("s_waitcnt vmcnt(6)\n\ts_barrier" ::: "memory");
      load_block(cur == 0 ? 2 : cur - 1, j + 2);
      const char* sb = smem + cur * kStage;
      cur = cur == 2 ? 0 : cur + 1;
      const bf16* Ks = (const bf16*)sb;
      const bf16* Ss = (const bf16*)(sb + kTile);
      // a key block wholly past this wavefront's last query adds nothing, and
      // its chunks were never stored (the dK/dV workgroup of those keys starts
      // at a later query): skip it
      if (64 * j > q0 + 32 * wv + 31) continue;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 sf = ds_frag<QW>(Ss, wv, kk * 16, lane);
#pragma unroll
        for (int x = 0; x < HB; ++x) dq[x] = mfma(tr_frag(Ks, x, kk * 16, lane), sf, dq[x]);
      }
    }
    wait_vmem();

    // QK-norm + RoPE backward of this lane's query, head h: with dqh the
    // gradient w.r.t. qh = R_t rho(q) and y = R_t^T qh = rho(q), the gradient
    // w.r.t. q is r (dy - y mean(dy y)), dy = R_t^T dqh.  Lanes l and l ^ 32
    // hold the two halves of the head row: element 32 x + 8 rg + 4 g + e is
    // dq[x][4 rg + e], so the pair (i, i + 64) is (x, x + 2) of one lane and
    // only the mean needs the partner lane.
    const bool live = qi < T;
    const float sc = -p.scale;  // the stored matrix is -dS
    const size_t n = tok0 + (live ? qi : 0);
    const int t = live ? qi : 0;
    const bf16* vrow = (const bf16*)p.q + n * p.ldq + h * HD;
    // dq[x] becomes dy of elements i (x < 2) and i + 64 (dq[x + 2]); ylo / yhi
    // hold y of the same elements
    f32x16 ylo[2], yhi[2];
    float dot = 0.f;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int i = 32 * x + 8 * rg + 4 * g;  // pairs i .. i + 3
        const f32x4 c01 = *reinterpret_cast<const f32x4*>(p.cs + 2 * ((size_t)t * 64 + i));
        const f32x4 c23 = *reinterpret_cast<const f32x4*>(p.cs + 2 * ((size_t)t * 64 + i) + 4);
        const f32x4 cv{c01.x, c01.z, c23.x, c23.z}, sv{c01.y, c01.w, c23.y, c23.w};
        const u32x2 a0 = *reinterpret_cast<const u32x2*>(vrow + i);
        const u32x2 a1 = *reinterpret_cast<const u32x2*>(vrow + i + 64);
        const f32x4 v0{bf16lo_to_f32(a0.x), bf16hi_to_f32(a0.x), bf16lo_to_f32(a0.y), bf16hi_to_f32(a0.y)};
        const f32x4 v1{bf16lo_to_f32(a1.x), bf16hi_to_f32(a1.x), bf16lo_to_f32(a1.y), bf16hi_to_f32(a1.y)};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * rg + e;
          const float g0 = dq[x][r] * sc, g1 = dq[x + 2][r] * sc;
          const float d0 = g0 * cv[e] + g1 * sv[e], d1 = g1 * cv[e] - g0 * sv[e];
          const float y0 = v0[e] * cv[e] + v1[e] * sv[e], y1 = v1[e] * cv[e] - v0[e] * sv[e];
          dq[x][r] = d0;
          dq[x + 2][r] = d1;
          ylo[x][r] = y0;
          yhi[x][r] = y1;
          dot = fmaf(d0, y0, fmaf(d1, y1, dot));
        }
      }
    dot += __shfl_xor(dot, 32, 64);
    dot *= 1.0f / 128.0f;
    if (live) {
      const float rr = p.rq[n * p.H + h];
      bf16* out = (bf16*)p.dq_pre + n * p.lddq_pre + h * HD;
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int i = 32 * x + 8 * rg + 4 * g;
          f32x4 lo, hi;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * rg + e;
            lo[e] = (dq[x][r] - ylo[x][r] * dot) * rr;
            hi[e] = (dq[x + 2][r] - yhi[x][r] * dot) * rr;
          }
          *reinterpret_cast<u32x2*>(out + i) = u32x2{pack_bf16x2(lo.x, lo.y), pack_bf16x2(lo.z, lo.w)};
          *reinterpret_cast<u32x2*>(out + i + 64) = u32x2{pack_bf16x2(hi.x, hi.y), pack_bf16x2(hi.z, hi.w)};
        }
    }
  }
}

// dK, dV with two wavefronts per 32 keys: 512 threads, 128 keys per
// workgroup.  Wavefronts p and p + 4 share a SIMD and own keys
// k0 + 32 p .. + 31:
//   the P wavefront (p) holds K: S = qh kh^T, P = exp2(S c - lse) (masked on
//     the diagonal and past T), dV += P^T dO; it hands P (the bf16 B operand
//     it built for dV) to its partner through LDS;
//   the dS wavefront (p + 4) holds -V: its dP accumulator starts at D and
//     ends at D - dP, -dS = P (D - dP) with the partner's P, dK' += (-dS)^T
//     qh; it stores -dS for the dQ kernel (lane-major chunks, ds_chunk).
// Each wavefront keeps one accumulator set (dV or dK, with K or -V: about
// half of what one wavefront holding both needs), so two share a SIMD and
// one's exponentials, products or LDS waits overlap the other's matrix
// products.
//
// Blocks of 64 queries (qh, dO tiles; lse, D) stream through three LDS
// stages; P goes through one of two exchange buffers.  One workgroup barrier
// per block, X_j: between X_{j-1} and X_j every wavefront issues the loads of
// block j + 1 (into the stage of block j - 2, whose last readers finished
// before X_{j-1}), then the P wavefront runs S, P (writing P_j) and dV of
// block j, the dS wavefront dS, dK of block j - 1 (reading P_{j-1}) and dP
// of block j.  At X_j each wavefront has waited for its own loads of block
// j + 1, so after it the whole block is in LDS; exchange buffer j & 1 is
// rewritten two blocks later, after every reader of P_j passed X_{j+1}.
//
// With dk_lp and rk (bf16, no key groups) the dS wavefront ends with the
// QK-norm + RoPE backward of its keys: after the last block the P wavefront
// writes K (kh) into the exchange buffers, now free, and the dS wavefront
// rotates dkh and kh back, forms the norm backward with its partner lane
// and writes the gradient w.r.t. the pre-norm k.
//
// LDS (bytes): qh tiles of the three stages [0, 48K), dO tiles [48K, 96K)
// (64 rows x 256 bytes, sw2 chunk swizzle), the lse and D vectors of stage st
// at 96K + 2K st and 1K beyond, the exchange buffers from 102K (buffer x,
// pair p, fragment f at 16K x + 4K p + 1K f, lane l's 16 bytes at 16 l).
// Each wavefront keeps the per-lane byte offsets of its fragment reads in
// registers and moves them to the next stage once per block (a uniform
// delta), so a read is one register plus an immediate offset.
constexpr uint32_t kPrTile = 64 * 128 * 2;
constexpr uint32_t kPrQ = 0, kPrO = 3 * kPrTile, kPrV = 6 * kPrTile, kPrX = kPrV + 3 * 2048;
constexpr uint32_t kPrBytes = kPrX + 2 * 16384;

__global__ void __launch_bounds__(512, 1) attn_bwd_dkdv_pair128(AttnArgs p) {
  constexpr int HD = 128, KS = 8, HB = 4;
  __shared__ __attribute__((aligned(1024))) char smem[kPrBytes];
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  const int T = p.T;
  const int nkb = gridDim.x;
  const int lin = xcd_block(blockIdx.x + nkb * blockIdx.y, nkb * gridDim.y);
  const int kbk = lin % nkb;  // key blocks of one (b, h) in turn, the longest first
  const int bh = lin / nkb, b = bh / p.H, h = bh % p.H;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pr = wv & 3;        // the pair, i.e. the 32 keys
  const bool pwave = wv < 4;    // the P wavefront of its pair (else the dS wavefront)
  const int g = lane >> 5, li = lane & 31;
  const int k0 = kbk * 128;
  const int wk = k0 + pr * 32;  // the pair's first key
  const int kj = wk + li;       // this lane's key
  const size_t tok0 = (size_t)b * T;
  const rsrc_t rq = make_rsrc((const bf16*)p.q + tok0 * p.ldq,
                              (uint32_t)(((size_t)(T - 1) * p.ldq + (size_t)p.H * HD) * 2));
  const rsrc_t ro = make_rsrc((const bf16*)p.dout + tok0 * p.lddo,
                              (uint32_t)(((size_t)(T - 1) * p.lddo + (size_t)p.H * HD) * 2));
  // wavefront 0 loads lse (base 2), wavefront 1 D
  const rsrc_t rv = make_rsrc(wv == 1 ? (const void*)(p.Dbuf + (size_t)bh * T) : (const void*)(p.lse + (size_t)bh * T),
                              (uint32_t)T * 4u);
  const long col = (long)h * HD;
  const int qb0 = k0 / 64;
  const int nb = (T + 63) / 64 - qb0;  // query blocks at or after the diagonal
  const float c = p.scale_log2;
  // the dS wavefront also finishes the QK-norm + RoPE backward of k
  const bool k_fused = p.dk_lp && p.rk && p.cs && p.G == 1;

  // this wavefront's loads of a block: slots wv and wv + 8 (4 rows each) of
  // the qh and dO tiles; wavefronts 0 and 1 also load a vector
  uint32_t toff_q[2], toff_o[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = (wv + 8 * i) * 4 + (lane >> 4);
    const int cc = (lane & 15) ^ sw2(row);
    toff_q[i] = (uint32_t)(((long)row * p.ldq + col + cc * 8) * 2);
    toff_o[i] = (uint32_t)(((long)row * p.lddo + col + cc * 8) * 2);
  }
  auto load_block = [&](int j) {
    const uint32_t st = (uint32_t)(j % 3);
    const int row0 = j < nb ? (qb0 + j) * 64 : T;  // blocks past the last read 0
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t slot = st * kPrTile + (uint32_t)(wv + 8 * i) * 1024u;
      const bool ok = row0 + (wv + 8 * i) * 4 + (lane >> 4) < T;
      dma16(rq, ok ? toff_q[i] + (uint32_t)(row0 * p.ldq * 2) : kOOB, lds0 + kPrQ + slot);
      dma16(ro, ok ? toff_o[i] + (uint32_t)(row0 * p.lddo * 2) : kOOB, lds0 + kPrO + slot);
    }
    if (wv < 2) {
      const int t = row0 + 4 * lane;
      dma16(rv, (lane < 16 && t < T) ? (uint32_t)t * 4u : kOOB, lds0 + kPrV + st * 2048u + (uint32_t)wv * 1024u);
    }
  };

  // Per-lane LDS byte offsets (see above): row fragment s of tile row li
  // (queries 0..31 of a block; +8 KB for 32..63) in this wavefront's row-read
  // tile (qh for the P wavefront, dO for the dS wavefront), stage of block j;
  // the two halves of transposed fragment x (reduction rows 0..15; +4 KB per
  // 16 rows) in its other tile, stage of block j - 1; its exchange slot
  // (buffer of block j for the P wavefront, of block j - 1 for the dS
  // wavefront); its vector (lse or D of queries 4 g .., stage of block j).
  uint32_t roff[KS], toff[HB][2], xoff, voff;
  {
    const uint32_t rbase = pwave ? kPrQ : kPrO, tbase = pwave ? kPrO : kPrQ + 2 * kPrTile;
#pragma unroll
    for (int s = 0; s < KS; ++s) roff[s] = rbase + (uint32_t)(li * 256 + (((2 * s + g) ^ sw2(li)) << 4));
    const int gi = lane >> 4, i = lane & 15, r = i >> 2, q = i & 3;
#pragma unroll
    for (int x = 0; x < HB; ++x)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int chunk = x * 4 + 2 * (gi & 1) + (q >> 1);
        const int kr = 4 * (gi >> 1) + r + 8 * hh;
        toff[x][hh] = tbase + (uint32_t)(kr * 256 + ((chunk ^ sw2(kr)) << 4) + 8 * (q & 1));
      }
    xoff = kPrX + (pwave ? 0u : 16384u) + (uint32_t)pr * 4096u + (uint32_t)lane * 16u;
    voff = kPrV + (pwave ? 0u : 1024u) + 16u * (uint32_t)g;
  }
  // move to block j: by one stage (back to the first after the third), and
  // the other exchange buffer.  The offsets pass through an empty asm, so
  // the compiler neither re-derives them per read nor keeps base + immediate
  // sums of its own.
  auto advance = [&](int j) __attribute__((always_inline)) {
    const uint32_t dst = (j % 3 == 0) ? (uint32_t)(-2 * (int)kPrTile) : kPrTile;  // row reads: stage of j
    // transposed reads: stage of block j (P wavefront) or j - 1 (dS wavefront)
    const uint32_t dtt = ((pwave ? j : j + 2) % 3 == 0) ? (uint32_t)(-2 * (int)kPrTile) : kPrTile;
    const uint32_t dv = (j % 3 == 0) ? (uint32_t)(-2 * 2048) : 2048u;
    // exchange buffer: of block j (P wavefront) or of block j - 1 (dS wavefront)
    const uint32_t dx = ((pwave ? j : j + 1) & 1) ? 16384u : (uint32_t)-16384;
#pragma unroll
    for (int s = 0; s < KS; ++s) roff[s] += dst;
#pragma unroll
    for (int x = 0; x < HB; ++x) { toff[x][0] += dtt; toff[x][1] += dtt; }
    voff += dv;
    xoff += dx;
    asm volatile("" : "+v"(roff[0]), "+v"(roff[1]), "+v"(roff[2]), "+v"(roff[3]), "+v"(roff[4]), "+v"(roff[5]),
                 "+v"(roff[6]), "+v"(roff[7]));
    asm volatile("" : "+v"(toff[0][0]), "+v"(toff[0][1]), "+v"(toff[1][0]), "+v"(toff[1][1]), "+v"(toff[2][0]),
                 "+v"(toff[2][1]), "+v"(toff[3][0]), "+v"(toff[3][1]), "+v"(xoff), "+v"(voff));
  };
  auto rowf = [&](uint32_t imm, int s) { return *reinterpret_cast<const bf16x8*>(smem + imm + roff[s]); };
  auto trf = [&](uint32_t imm, int x) {
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)(smem + imm + toff[x][0]));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)(smem + imm + toff[x][1]));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto vec4 = [&](uint32_t imm) { return *reinterpret_cast<const f32x4*>(smem + imm + voff); };

  load_block(0);

  if (pwave) {
    // ------------------------------------------------------------ P wavefront
    const bf16* kp = (const bf16*)p.k + tok0 * p.ldk + (h / p.G) * HD;
    bf16x8 kf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s)
      kf[s] = kj < T ? *reinterpret_cast<const bf16x8*>(kp + (size_t)kj * p.ldk + s * 16 + g * 8) : bf16x8{};
    // wait for K here: the compiler does not see the waits of the asm below,
    // and would otherwise wait for all loads (those of the next block too) at
    // the first use of K inside the loop, every block
#pragma unroll
    for (int s = 0; s < KS; ++s) asm volatile("" ::"v"(kf[s]));
    f32x16 dv[HB];
#pragma unroll
    for (int x = 0; x < HB; ++x) dv[x] = f32x16{};
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");  // X_{-1}: block 0 landed
    // one block: loads of block j + 1; S of both halves (fragment reads
    // first, the two accumulation chains interleaved), P = exp2(S c - lse)
    // written to the exchange buffer, dV += P^T dO
    auto seg = [&](auto masked, int j) __attribute__((always_inline)) {
      constexpr bool MASKED = decltype(masked)::value;
      if (j > 0) advance(j);
      load_block(j + 1);
      bf16x8 fq[2][KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        fq[0][s] = rowf(0u, s);
        fq[1][s] = rowf(8192u, s);
      }
      __builtin_amdgcn_sched_barrier(0);
      f32x16 S[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        S[0] = mfma(fq[0][s], kf[s], S[0]);
        S[1] = mfma(fq[1][s], kf[s], S[1]);
      }
      __builtin_amdgcn_sched_barrier(0);
      const int qbase = (qb0 + j) * 64;
      bf16x8 pf[4];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        f32x16 P;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const f32x4 l4 = vec4((uint32_t)(mi * 32 + 8 * rb) * 4u);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * rb + e;
            float pv = ex2(fmaf(S[mi][r], c, -l4[e]));
            if constexpr (MASKED) {
              const int q = qbase + mi * 32 + 8 * rb + 4 * g + e;
              pv = (q < kj || q >= T) ? 0.f : pv;
            }
            P[r] = pv;
          }
        }
        pf[2 * mi] = pack8(P, 0);
        pf[2 * mi + 1] = pack8(P, 1);
#pragma unroll
        for (int t = 0; t < 2; ++t)
          *reinterpret_cast<bf16x8*>(smem + (uint32_t)(2 * mi + t) * 1024u + xoff) = pf[2 * mi + t];
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int x = 0; x < HB; ++x)
            dv[x] = mfma(trf((uint32_t)(mi * 32 + t * 16) * 256u, x), pf[2 * mi + t], dv[x]);
      // X_j: the P writes are done and this wavefront's loads of block j + 1 landed
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    // the first two blocks meet the diagonal, a block j with (qb0 + j + 1) *
    // 64 > T meets the end: masked ranges are a prefix and a suffix
    const int j_end = min(nb, max(2, T / 64 - qb0));
    int j = 0;
    for (; j < min(2, nb); ++j) seg(std::true_type{}, j);
    for (; j < j_end; ++j) seg(std::false_type{}, j);
    for (; j < nb; ++j) seg(std::true_type{}, j);
    // the dS wavefront's last block (no loads: those of block nb + 1 read 0)
    load_block(j + 1);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    if (k_fused) {
      // K for the dS partner's QK-norm + RoPE backward, through the exchange
      // buffers (read for the last time before the barrier above): pair pr,
      // key row li (256 bytes), 16-byte chunk c of the row at slot c ^ (li & 15)
#pragma unroll
      for (int s = 0; s < KS; ++s)
        *reinterpret_cast<bf16x8*>(smem + kPrX + (uint32_t)pr * 8192u + (uint32_t)li * 256u +
                                   ((uint32_t)((2 * s + g) ^ (li & 15)) << 4)) = kf[s];
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    if (kj >= T) return;
    bf16* dvq = (bf16*)p.dv + (tok0 + kj) * p.lddv + h * HD;
#pragma unroll
    for (int x = 0; x < HB; ++x)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        u32x2 w;
        w.x = pack_bf16x2(dv[x][rg * 4 + 0], dv[x][rg * 4 + 1]);
        w.y = pack_bf16x2(dv[x][rg * 4 + 2], dv[x][rg * 4 + 3]);
        *reinterpret_cast<u32x2*>(dvq + x * 32 + 8 * rg + 4 * g) = w;
      }
  } else {
    // ----------------------------------------------------------- dS wavefront
    const bf16* vp = (const bf16*)p.v + tok0 * p.ldv + (h / p.G) * HD;
    bf16x8 vn[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 v = kj < T ? *reinterpret_cast<const bf16x8*>(vp + (size_t)kj * p.ldv + s * 16 + g * 8) : bf16x8{};
      vn[s] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, v) ^ 0x80008000u);  // -V
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) asm volatile("" ::"v"(vn[s]));  // wait for V here (see the P wavefront)
    f32x16 dk[HB];
#pragma unroll
    for (int x = 0; x < HB; ++x) dk[x] = f32x16{};
    f32x16 Pd[2];  // D - dP of the previous block, per half
    const long Tp = p.tpad;
    const rsrc_t rds = make_rsrc((const bf16*)p.dsT + (size_t)bh * Tp * Tp, (uint32_t)(Tp * Tp * 2));
    const uint32_t ds_lane = (uint32_t)lane * 16u;
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");  // X_{-1}: block 0 landed
    // -dS = P (D - dP) of block jp from the partner's P, stored, then
    // dK' += (-dS)^T qh
    auto dsk = [&](int jp) __attribute__((always_inline)) {
      const int qbase = (qb0 + jp) * 64;
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        bf16x8 sf[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(smem + (uint32_t)(2 * mi + t) * 1024u + xoff);
          // fragment t holds accumulator registers 8 t .. 8 t + 7, two per dword
          u32x4 o;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            o[q] = pack_bf16x2(bf16lo_to_f32(w[q]) * Pd[mi][8 * t + 2 * q],
                               bf16hi_to_f32(w[q]) * Pd[mi][8 * t + 2 * q + 1]);
          sf[t] = __builtin_bit_cast(bf16x8, o);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, sf[t]), rds, ds_lane,
                                                 (int)ds_chunk(Tp, wk >> 5, (qbase + 32 * mi) >> 5, t), 2);
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int x = 0; x < HB; ++x) dk[x] = mfma(trf((uint32_t)(mi * 32 + t * 16) * 256u, x), sf[t], dk[x]);
      }
    };
    int j = 0;
    for (; j < nb; ++j) {
      // one block: loads of block j + 1, dS and dK of block j - 1, D - dP of block j
      if (j > 0) advance(j);
      load_block(j + 1);
      if (j > 0) dsk(j - 1);
      __builtin_amdgcn_sched_barrier(0);
      // D - dP of both halves: fragment and D reads first, then the two
      // accumulation chains interleaved
      bf16x8 fo[2][KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        fo[0][s] = rowf(0u, s);
        fo[1][s] = rowf(8192u, s);
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const f32x4 d4 = vec4((uint32_t)(mi * 32 + 8 * rb) * 4u);
          Pd[mi][4 * rb + 0] = d4.x;
          Pd[mi][4 * rb + 1] = d4.y;
          Pd[mi][4 * rb + 2] = d4.z;
          Pd[mi][4 * rb + 3] = d4.w;
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        Pd[0] = mfma(fo[0][s], vn[s], Pd[0]);
        Pd[1] = mfma(fo[1][s], vn[s], Pd[1]);
      }
      // X_j: this wavefront's loads of block j + 1 landed; the only vector
      // memory operations issued after them are the 4 dS stores of block j - 1
      if (j > 0) asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    }
    advance(j);
    load_block(j + 1);
    // the RoPE-table entries and 1/rms of this lane's key for the fused
    // QK-norm + RoPE backward below, loaded under the last block's dK product
    // (the wait after it covers them)
    const bool live = kj < T;
    const int t = live ? kj : 0;
    float rr = 0.f;
    f32x4 cv[2][4], sv[2][4];
    if (k_fused) {
      rr = live ? p.rk[(tok0 + t) * p.H + h] : 0.f;
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int i = 32 * x + 8 * rg + 4 * g;
          const f32x4 c01 = *reinterpret_cast<const f32x4*>(p.cs + 2 * ((size_t)t * 64 + i));
          const f32x4 c23 = *reinterpret_cast<const f32x4*>(p.cs + 2 * ((size_t)t * 64 + i) + 4);
          cv[x][rg] = f32x4{c01.x, c01.z, c23.x, c23.z};
          sv[x][rg] = f32x4{c01.y, c01.w, c23.y, c23.w};
        }
    }
    dsk(j - 1);
    asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
    wait_vmem();
    const float sc = -p.scale;  // dK' = -dK
    if (k_fused) {
      // QK-norm + RoPE backward of this lane's key (as the dQ kernel does for
      // q): with dkh the gradient w.r.t. kh = R_t rho(k) and y = R_t^T kh,
      // the gradient w.r.t. k is r (dy - y mean(dy y)), dy = R_t^T dkh.
      // Element 32 x + 8 rg + 4 g + e is dk[x][4 rg + e]; the pair (i, i + 64)
      // is (x, x + 2) of one lane and the mean needs the partner lane.  kh
      // comes from the P partner through LDS.
      asm volatile("s_barrier" ::: "memory");  // the P partner's K is in LDS
      const char* krow = smem + kPrX + (uint32_t)pr * 8192u + (uint32_t)li * 256u;
      float dot = 0.f;
      f32x16 ylo[2], yhi[2];
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int c0 = 4 * x + rg, c1 = 4 * (x + 2) + rg;  // chunks of elements i and i + 64
          const u32x2 a0 = *reinterpret_cast<const u32x2*>(krow + ((uint32_t)(c0 ^ (li & 15)) << 4) + 8 * g);
          const u32x2 a1 = *reinterpret_cast<const u32x2*>(krow + ((uint32_t)(c1 ^ (li & 15)) << 4) + 8 * g);
          const f32x4 v0{bf16lo_to_f32(a0.x), bf16hi_to_f32(a0.x), bf16lo_to_f32(a0.y), bf16hi_to_f32(a0.y)};
          const f32x4 v1{bf16lo_to_f32(a1.x), bf16hi_to_f32(a1.x), bf16lo_to_f32(a1.y), bf16hi_to_f32(a1.y)};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * rg + e;
            const float cc = cv[x][rg][e], ss = sv[x][rg][e];
            const float g0 = dk[x][r] * sc, g1 = dk[x + 2][r] * sc;
            const float d0 = g0 * cc + g1 * ss, d1 = g1 * cc - g0 * ss;
            const float y0 = v0[e] * cc + v1[e] * ss, y1 = v1[e] * cc - v0[e] * ss;
            dk[x][r] = d0;
            dk[x + 2][r] = d1;
            ylo[x][r] = y0;
            yhi[x][r] = y1;
            dot = fmaf(d0, y0, fmaf(d1, y1, dot));
          }
        }
      dot += __shfl_xor(dot, 32, 64);
      dot *= 1.0f / 128.0f;
      if (!live) return;
      bf16* out = (bf16*)p.dk_lp + (tok0 + kj) * p.lddk_lp + h * HD;
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int i = 32 * x + 8 * rg + 4 * g;
          f32x4 lo, hi;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * rg + e;
            lo[e] = (dk[x][r] - ylo[x][r] * dot) * rr;
            hi[e] = (dk[x + 2][r] - yhi[x][r] * dot) * rr;
          }
          *reinterpret_cast<u32x2*>(out + i) = u32x2{pack_bf16x2(lo.x, lo.y), pack_bf16x2(lo.z, lo.w)};
          *reinterpret_cast<u32x2*>(out + i + 64) = u32x2{pack_bf16x2(hi.x, hi.y), pack_bf16x2(hi.z, hi.w)};
        }
      return;
    }
    if (kj >= T) return;
    if (p.dk_lp) {
      bf16* dkp = (bf16*)p.dk_lp + (tok0 + kj) * p.lddk_lp + h * HD;
#pragma unroll
      for (int x = 0; x < HB; ++x)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg)
          *reinterpret_cast<u32x2*>(dkp + x * 32 + 8 * rg + 4 * g) =
              u32x2{pack_bf16x2(dk[x][rg * 4 + 0] * sc, dk[x][rg * 4 + 1] * sc),
                    pack_bf16x2(dk[x][rg * 4 + 2] * sc, dk[x][rg * 4 + 3] * sc)};
      return;
    }
    float* dkp = p.dk32 + (tok0 + kj) * p.lddk + h * HD;
#pragma unroll
    for (int x = 0; x < HB; ++x)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        f32x4 w{dk[x][rg * 4 + 0] * sc, dk[x][rg * 4 + 1] * sc, dk[x][rg * 4 + 2] * sc, dk[x][rg * 4 + 3] * sc};
        *reinterpret_cast<f32x4*>(dkp + x * 32 + 8 * rg + 4 * g) = w;
      }
  }
}

// ------------------------------------------------------------------ backward: D
template <class T>
__global__ void __launch_bounds__(256) attn_bwd_pre(AttnArgs p, int hd) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);  // (b, t, h) flattened
  const int lane = threadIdx.x & 63;
  const int N = p.B * p.T;
  if (row >= N * p.H) return;
  const int n = row / p.H, h = row % p.H;
  const T* o = (const T*)p.o + (size_t)n * p.ldo + h * hd;
  const T* d = (const T*)p.dout + (size_t)n * p.lddo + h * hd;
  float s = 0.f;
  for (int e = lane; e < hd; e += 64) s += to_f32(o[e]) * to_f32(d[e]);
  s = wave_sum(s);
  const int b = n / p.T, t = n % p.T;
  if (lane == 0) p.Dbuf[((size_t)b * p.H + h) * p.T + t] = s;
}

// ------------------------------------------------------------------ backward: dK, dV
template <int HD>
__global__ void __launch_bounds__(256) attn_bwd_dkdv_mfma(AttnArgs p) {
  constexpr int KS = HD / 16, HB = HD / 32;
  __shared__ __attribute__((aligned(16))) bf16 Qs[64 * (HD + 8)];
  __shared__ __attribute__((aligned(16))) bf16 Qt[HD * (64 + 4)];
  __shared__ __attribute__((aligned(16))) bf16 Ds[64 * (HD + 8)];
  __shared__ __attribute__((aligned(16))) bf16 Dt[HD * (64 + 4)];
  __shared__ float lse_s[64], D_s[64];

  const int T = p.T;
  const int nkb = (T + 127) / 128;
  const int kb = blockIdx.x;  // low key blocks have the most queries: first
  const int bh = blockIdx.y, b = bh / p.H, h = bh % p.H;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 5, li = lane & 31;
  const int k0 = kb * 128;
  const int kj = k0 + wv * 32 + li;
  const size_t tok0 = (size_t)b * T;
  (void)nkb;

  const bf16* qp = (const bf16*)p.q + tok0 * p.ldq + h * HD;
  const bf16* kp = (const bf16*)p.k + tok0 * p.ldk + (h / p.G) * HD;
  const bf16* vp = (const bf16*)p.v + tok0 * p.ldv + (h / p.G) * HD;
  const bf16* dop = (const bf16*)p.dout + tok0 * p.lddo + h * HD;
  const float* lsep = p.lse + (size_t)bh * T;
  const float* Dp = p.Dbuf + (size_t)bh * T;

  bf16x8 kf[KS], vf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    kf[s] = kj < T ? *reinterpret_cast<const bf16x8*>(kp + (size_t)kj * p.ldk + s * 16 + g * 8) : bf16x8{};
    vf[s] = kj < T ? *reinterpret_cast<const bf16x8*>(vp + (size_t)kj * p.ldv + s * 16 + g * 8) : bf16x8{};
  }
  f32x16 dk[HB], dv[HB];
#pragma unroll
  for (int x = 0; x < HB; ++x) { dk[x] = f32x16{}; dv[x] = f32x16{}; }

  const int nqb = (T + 63) / 64;
  const int qb0 = k0 / 64;
  const int wk_min = k0 + wv * 32;

  KvStage<HD> sq, sd;
  sq.load(qp, p.ldq, qb0 * 64, T);
  sd.load(dop, p.lddo, qb0 * 64, T);
  for (int qb = qb0; qb < nqb; ++qb) {
    const int qbase = qb * 64;
    __syncthreads();
    sq.store_rows(Qs);
    sq.store_cols(Qt);
    sd.store_rows(Ds);
    sd.store_cols(Dt);
    if (threadIdx.x < 64) {
      const int t = qbase + threadIdx.x;
      lse_s[threadIdx.x] = t < T ? lsep[t] : 0.f;
      D_s[threadIdx.x] = t < T ? Dp[t] : 0.f;
    }
    __syncthreads();
    if (qb + 1 < nqb) {
      sq.load(qp, p.ldq, (qb + 1) * 64, T);
      sd.load(dop, p.lddo, (qb + 1) * 64, T);
    }
    if (qbase + 63 < wk_min) continue;  // every query of this block precedes this wave's keys

    f32x16 sacc[2], pacc[2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
      sacc[mi] = f32x16{};
      pacc[mi] = f32x16{};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(Qs + (mi * 32 + li) * (HD + 8) + s * 16 + g * 8);
        sacc[mi] = mfma(qa, kf[s], sacc[mi]);
        const bf16x8 da = *reinterpret_cast<const bf16x8*>(Ds + (mi * 32 + li) * (HD + 8) + s * 16 + g * 8);
        pacc[mi] = mfma(da, vf[s], pacc[mi]);
      }
    }
    const bool need_mask = (qbase < wk_min + 31) || (qbase + 64 > T);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ql = mi * 32 + acc_row(r, g);
        float pr = exp2f(sacc[mi][r] * p.scale_log2 - lse_s[ql]);
        if (need_mask) {
          const int q = qbase + ql;
          if (q < kj || q >= T) pr = 0.f;
        }
        sacc[mi][r] = pr;                       // P
        pacc[mi][r] = pr * (pacc[mi][r] - D_s[ql]);  // dS
      }
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8 pf = pack8(sacc[mi], t);
        const bf16x8 sf = pack8(pacc[mi], t);
#pragma unroll
        for (int x = 0; x < HB; ++x) {
          const bf16x8 dot = read_t8(Dt, x * 32 + li, mi * 32 + t * 16 + 4 * g);
          dv[x] = mfma(dot, pf, dv[x]);
          const bf16x8 qt = read_t8(Qt, x * 32 + li, mi * 32 + t * 16 + 4 * g);
          dk[x] = mfma(qt, sf, dk[x]);
        }
      }
  }
  if (kj >= T) return;
  const float sc = p.scale;
  float* dkp = p.dk32 + (tok0 + kj) * p.lddk + h * HD;
#pragma unroll
  for (int x = 0; x < HB; ++x)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      f32x4 w{dk[x][rg * 4 + 0] * sc, dk[x][rg * 4 + 1] * sc, dk[x][rg * 4 + 2] * sc, dk[x][rg * 4 + 3] * sc};
      *reinterpret_cast<f32x4*>(dkp + x * 32 + 8 * rg + 4 * g) = w;
    }
  bf16* dvp = (bf16*)p.dv + (tok0 + kj) * p.lddv + h * HD;
#pragma unroll
  for (int x = 0; x < HB; ++x)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      u32x2 w;
      w.x = pack_bf16x2(dv[x][rg * 4 + 0], dv[x][rg * 4 + 1]);
      w.y = pack_bf16x2(dv[x][rg * 4 + 2], dv[x][rg * 4 + 3]);
      *reinterpret_cast<u32x2*>(dvp + x * 32 + 8 * rg + 4 * g) = w;
    }
}

// ------------------------------------------------------------------ backward: dQ
template <int HD>
__global__ void __launch_bounds__(256) attn_bwd_dq_mfma(AttnArgs p) {
  constexpr int KS = HD / 16, HB = HD / 32;
  __shared__ __attribute__((aligned(16))) bf16 Ks[64 * (HD + 8)];
  __shared__ __attribute__((aligned(16))) bf16 Kt[HD * (64 + 4)];
  __shared__ __attribute__((aligned(16))) bf16 Vs[64 * (HD + 8)];

  const int T = p.T;
  const int nqb = gridDim.x;  // (T + 127) / 128
  const int lin = xcd_block(blockIdx.x + nqb * blockIdx.y, nqb * gridDim.y);
  const int qb = nqb - 1 - lin % nqb;  // query blocks of one (b, h) in turn on one XCD, the longest first
  const int bh = lin / nqb, b = bh / p.H, h = bh % p.H;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 5, li = lane & 31;
  const int q0 = qb * 128;
  const int qi = q0 + wv * 32 + li;
  const size_t tok0 = (size_t)b * T;

  const bf16* qp = (const bf16*)p.q + tok0 * p.ldq + h * HD;
  const bf16* kp = (const bf16*)p.k + tok0 * p.ldk + (h / p.G) * HD;
  const bf16* vp = (const bf16*)p.v + tok0 * p.ldv + (h / p.G) * HD;
  const bf16* dop = (const bf16*)p.dout + tok0 * p.lddo + h * HD;

  bf16x8 qf[KS], df[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    qf[s] = qi < T ? *reinterpret_cast<const bf16x8*>(qp + (size_t)qi * p.ldq + s * 16 + g * 8) : bf16x8{};
    df[s] = qi < T ? *reinterpret_cast<const bf16x8*>(dop + (size_t)qi * p.lddo + s * 16 + g * 8) : bf16x8{};
  }
  const float lse_l = qi < T ? p.lse[(size_t)bh * T + qi] : 0.f;
  const float Dl = qi < T ? p.Dbuf[(size_t)bh * T + qi] : 0.f;

  f32x16 dq[HB];
#pragma unroll
  for (int x = 0; x < HB; ++x) dq[x] = f32x16{};

  const int q_last = min(T - 1, q0 + 127);
  const int nkv = q_last / 64 + 1;
  const int wq_min = q0 + wv * 32, wq_max = wq_min + 31;

  KvStage<HD> sk, sv;
  sk.load(kp, p.ldk, 0, T);
  sv.load(vp, p.ldv, 0, T);
  for (int kb = 0; kb < nkv; ++kb) {
    __syncthreads();
    sk.store_rows(Ks);
    sk.store_cols(Kt);
    sv.store_rows(Vs);
    __syncthreads();
    if (kb + 1 < nkv) {
      sk.load(kp, p.ldk, (kb + 1) * 64, T);
      sv.load(vp, p.ldv, (kb + 1) * 64, T);
    }
    const int kbase = kb * 64;
    if (kbase > wq_max) continue;

    f32x16 sacc[2], pacc[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      sacc[kk] = f32x16{};
      pacc[kk] = f32x16{};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Ks + (kk * 32 + li) * (HD + 8) + s * 16 + g * 8);
        sacc[kk] = mfma(ka, qf[s], sacc[kk]);
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(Vs + (kk * 32 + li) * (HD + 8) + s * 16 + g * 8);
        pacc[kk] = mfma(va, df[s], pacc[kk]);
      }
    }
    const bool need_mask = (kbase + 63 > wq_min) || (kbase + 64 > T);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pr = exp2f(sacc[kk][r] * p.scale_log2 - lse_l);
        if (need_mask) {
          const int key = kbase + kk * 32 + acc_row(r, g);
          if (key > qi || key >= T) pr = 0.f;
        }
        pacc[kk][r] = pr * (pacc[kk][r] - Dl);  // dS^T
      }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8 sf = pack8(pacc[kk], t);
#pragma unroll
        for (int x = 0; x < HB; ++x) {
          const bf16x8 kt = read_t8(Kt, x * 32 + li, kk * 32 + t * 16 + 4 * g);
          dq[x] = mfma(kt, sf, dq[x]);
        }
      }
  }
  if (qi >= T) return;
  const float sc = p.scale;
  float* dqp = p.dq32 + (tok0 + qi) * p.lddq + h * HD;
#pragma unroll
  for (int x = 0; x < HB; ++x)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      f32x4 w{dq[x][rg * 4 + 0] * sc, dq[x][rg * 4 + 1] * sc, dq[x][rg * 4 + 2] * sc, dq[x][rg * 4 + 3] * sc};
      *reinterpret_cast<f32x4*>(dqp + x * 32 + 8 * rg + 4 * g) = w;
    }
}

// ------------------------------------------------------------------ fp32 SIMT path
// One wavefront per (b, h, query); lanes own head-dim elements e and e + 64.
template <class T>
__global__ void __launch_bounds__(256) attn_fwd_simt(AttnArgs p, int hd) {
  const long wid = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int T_ = p.T;
  if (wid >= (long)p.B * p.H * T_) return;
  const int qi = wid % T_;
  const int bh = wid / T_, b = bh / p.H, h = bh % p.H;
  const size_t tok0 = (size_t)b * T_;
  const T* qrow = (const T*)p.q + (tok0 + qi) * p.ldq + h * hd;
  const float sc = p.scale;
  float q0 = lane < hd ? to_f32(qrow[lane]) : 0.f, q1 = lane + 64 < hd ? to_f32(qrow[lane + 64]) : 0.f;
  float a0 = 0.f, a1 = 0.f, m = -INFINITY, l = 0.f;
  for (int j = 0; j <= qi; ++j) {
    const T* kr = (const T*)p.k + (tok0 + j) * p.ldk + (h / p.G) * hd;
    const T* vr = (const T*)p.v + (tok0 + j) * p.ldv + (h / p.G) * hd;
    float s = (lane < hd ? q0 * to_f32(kr[lane]) : 0.f) + (lane + 64 < hd ? q1 * to_f32(kr[lane + 64]) : 0.f);
    s = wave_sum(s) * sc;
    const float mn = fmaxf(m, s);
    const float al = expf(m - mn), pe = expf(s - mn);
    l = l * al + pe;
    a0 = a0 * al + pe * (lane < hd ? to_f32(vr[lane]) : 0.f);
    a1 = a1 * al + pe * (lane + 64 < hd ? to_f32(vr[lane + 64]) : 0.f);
    m = mn;
  }
  T* orow = (T*)p.o + (tok0 + qi) * p.ldo + h * hd;
  if (lane < hd) orow[lane] = from_f32<T>(a0 / l);
  if (lane + 64 < hd) orow[lane + 64] = from_f32<T>(a1 / l);
  if (lane == 0) p.lse[(size_t)bh * T_ + qi] = m + logf(l);
}

template <class T>
__global__ void __launch_bounds__(256) attn_bwd_dq_simt(AttnArgs p, int hd) {
  const long wid = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int T_ = p.T;
  if (wid >= (long)p.B * p.H * T_) return;
  const int qi = wid % T_;
  const int bh = wid / T_, b = bh / p.H, h = bh % p.H;
  const size_t tok0 = (size_t)b * T_;
  const T* qrow = (const T*)p.q + (tok0 + qi) * p.ldq + h * hd;
  const T* drow = (const T*)p.dout + (tok0 + qi) * p.lddo + h * hd;
  const bool e0 = lane < hd, e1 = lane + 64 < hd;
  const float q0 = e0 ? to_f32(qrow[lane]) : 0.f, q1 = e1 ? to_f32(qrow[lane + 64]) : 0.f;
  const float d0 = e0 ? to_f32(drow[lane]) : 0.f, d1 = e1 ? to_f32(drow[lane + 64]) : 0.f;
  const float lse = p.lse[(size_t)bh * T_ + qi], Dq = p.Dbuf[(size_t)bh * T_ + qi];
  const float sc = p.scale;
  float g0 = 0.f, g1 = 0.f;
  for (int j = 0; j <= qi; ++j) {
    const T* kr = (const T*)p.k + (tok0 + j) * p.ldk + (h / p.G) * hd;
    const T* vr = (const T*)p.v + (tok0 + j) * p.ldv + (h / p.G) * hd;
    const float k0 = e0 ? to_f32(kr[lane]) : 0.f, k1 = e1 ? to_f32(kr[lane + 64]) : 0.f;
    const float v0 = e0 ? to_f32(vr[lane]) : 0.f, v1 = e1 ? to_f32(vr[lane + 64]) : 0.f;
    const float s = wave_sum(q0 * k0 + q1 * k1) * sc;
    const float dp = wave_sum(d0 * v0 + d1 * v1);
    const float ds = expf(s - lse) * (dp - Dq);
    g0 += ds * k0;
    g1 += ds * k1;
  }
  float* o = p.dq32 + (tok0 + qi) * p.lddq + h * hd;
  if (e0) o[lane] = g0 * sc;
  if (e1) o[lane + 64] = g1 * sc;
}

template <class T>
__global__ void __launch_bounds__(256) attn_bwd_dkdv_simt(AttnArgs p, int hd) {
  const long wid = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int T_ = p.T;
  if (wid >= (long)p.B * p.H * T_) return;
  const int kj = wid % T_;
  const int bh = wid / T_, b = bh / p.H, h = bh % p.H;
  const size_t tok0 = (size_t)b * T_;
  const bool e0 = lane < hd, e1 = lane + 64 < hd;
  const T* kr = (const T*)p.k + (tok0 + kj) * p.ldk + (h / p.G) * hd;
  const T* vr = (const T*)p.v + (tok0 + kj) * p.ldv + (h / p.G) * hd;
  const float k0 = e0 ? to_f32(kr[lane]) : 0.f, k1 = e1 ? to_f32(kr[lane + 64]) : 0.f;
  const float v0 = e0 ? to_f32(vr[lane]) : 0.f, v1 = e1 ? to_f32(vr[lane + 64]) : 0.f;
  const float sc = p.scale;
  float gk0 = 0.f, gk1 = 0.f, gv0 = 0.f, gv1 = 0.f;
  for (int i = kj; i < T_; ++i) {
    const T* qrow = (const T*)p.q + (tok0 + i) * p.ldq + h * hd;
    const T* drow = (const T*)p.dout + (tok0 + i) * p.lddo + h * hd;
    const float q0 = e0 ? to_f32(qrow[lane]) : 0.f, q1 = e1 ? to_f32(qrow[lane + 64]) : 0.f;
    const float d0 = e0 ? to_f32(drow[lane]) : 0.f, d1 = e1 ? to_f32(drow[lane + 64]) : 0.f;
    const float s = wave_sum(q0 * k0 + q1 * k1) * sc;
    const float pr = expf(s - p.lse[(size_t)bh * T_ + i]);
    const float dp = wave_sum(d0 * v0 + d1 * v1);
    const float ds = pr * (dp - p.Dbuf[(size_t)bh * T_ + i]);
    gv0 += pr * d0; gv1 += pr * d1;
    gk0 += ds * q0; gk1 += ds * q1;
  }
  float* ko = p.dk32 + (tok0 + kj) * p.lddk + h * hd;
  T* vo = (T*)p.dv + (tok0 + kj) * p.lddv + h * hd;
  if (e0) { ko[lane] = gk0 * sc; vo[lane] = from_f32<T>(gv0); }
  if (e1) { ko[lane + 64] = gk1 * sc; vo[lane + 64] = from_f32<T>(gv1); }
}

// ------------------------------------------------------------------ launchers
int launch_attn_fwd(AttnArgs p, int hd, int dtype, hipStream_t s) {
  p.scale = 1.0f / sqrtf((float)hd);
  p.scale_log2 = p.scale * kLog2e;
  if (p.B * p.H * p.T == 0) return 0;
  if (dtype == 0) {
    dim3 grid((p.T + 127) / 128, p.B * p.H);
    if (hd == 128) attn_fwd128<<<grid, 256, 0, s>>>(p);
    else if (hd == 64) attn_fwd_mfma<64><<<grid, 256, 0, s>>>(p);
    else return 7;
  } else {
    const long waves = (long)p.B * p.H * p.T;
    attn_fwd_simt<float><<<(unsigned)((waves + 3) / 4), 256, 0, s>>>(p, hd);
  }
  NC_LAUNCH_CHECK();
  return 0;
}

int launch_attn_bwd(AttnArgs p, int hd, int dtype, hipStream_t s) {
  p.scale = 1.0f / sqrtf((float)hd);
  p.scale_log2 = p.scale * kLog2e;
  if (p.B * p.H * p.T == 0) return 0;
  const long rows = (long)p.B * p.T * p.H;
  if (dtype == 0) {
    dim3 gk((p.T + 127) / 128, p.B * p.H);
    dim3 gq((p.T + 127) / 128, p.B * p.H);
    if (hd == 128) {
      // D, then dK/dV (which stores dS), then dQ from the stored dS
      if (!p.dsT || p.tpad != attn_ds_pad(p.T)) return NC_ERR_WORKSPACE;
      if (!p.dq_pre || !p.rq || !p.cs) return NC_ERR_NULL;
      if (p.tpad > kMaxDsPad) return NC_ERR_UNSUPPORTED;  // one (b, h) block of dS must stay below 2 GiB
      attn_bwd_D128<<<(unsigned)((rows + 15) / 16), 256, 0, s>>>(p);
      attn_bwd_dkdv_pair128<<<gk, 512, 0, s>>>(p);
      attn_bwd_dq_ds128<<<dim3(((p.T + kDqQueries - 1) / kDqQueries + 1) / 2, p.B * p.H), 512, 0, s>>>(p);
    } else if (hd == 64) {
      attn_bwd_pre<bf16><<<(unsigned)((rows + 3) / 4), 256, 0, s>>>(p, hd);
      attn_bwd_dkdv_mfma<64><<<gk, 256, 0, s>>>(p);
      attn_bwd_dq_mfma<64><<<gq, 256, 0, s>>>(p);
    } else {
      return 7;
    }
  } else {
    attn_bwd_pre<float><<<(unsigned)((rows + 3) / 4), 256, 0, s>>>(p, hd);
    const long waves = (long)p.B * p.H * p.T;
    attn_bwd_dq_simt<float><<<(unsigned)((waves + 3) / 4), 256, 0, s>>>(p, hd);
    attn_bwd_dkdv_simt<float><<<(unsigned)((waves + 3) / 4), 256, 0, s>>>(p, hd);
  }
  NC_LAUNCH_CHECK();
  return 0;
}

// Grouped-query attention backward: the gradient of a shared key/value head
// is the sum over the G query heads that read it (fixed order g = 0..G-1).
// dk_q, dv_q hold one gradient per query head; dk (fp32) and dv (element
// type) one per key/value head.
template <class T>
__global__ void __launch_bounds__(256) kv_group_sum_kernel(const float* __restrict__ dk_q, long ldq_k,
                                                           const T* __restrict__ dv_q, long ldq_v,
                                                           float* __restrict__ dk, long ldk, T* __restrict__ dv,
                                                           long ldv, long N, int Hk, int G, int hd) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  const long per = (long)Hk * hd;
  if (i >= N * per) return;
  const long n = i / per;
  const int c = (int)(i - n * per);  // kv head * hd + e
  const int hk = c / hd, e = c - hk * hd;
  float sk = 0.f, sv = 0.f;
  for (int g = 0; g < G; ++g) {
    const long col = (long)(hk * G + g) * hd + e;
    sk += dk_q[n * ldq_k + col];
    sv += to_f32(dv_q[n * ldq_v + col]);
  }
  dk[n * ldk + c] = sk;
  dv[n * ldv + c] = from_f32<T>(sv);
}

int launch_kv_group_sum(const float* dk_q, long ldq_k, const void* dv_q, long ldq_v, float* dk, long ldk, void* dv,
                        long ldv, long N, int Hk, int G, int hd, int dtype, hipStream_t s) {
  const long total = N * Hk * hd;
  if (total == 0) return 0;
  const unsigned grid = (unsigned)((total + 255) / 256);
  if (dtype == 0)
    kv_group_sum_kernel<bf16><<<grid, 256, 0, s>>>(dk_q, ldq_k, (const bf16*)dv_q, ldq_v, dk, ldk, (bf16*)dv, ldv,
                                                   N, Hk, G, hd);
  else
    kv_group_sum_kernel<float><<<grid, 256, 0, s>>>(dk_q, ldq_k, (const float*)dv_q, ldq_v, dk, ldk, (float*)dv,
                                                    ldv, N, Hk, G, hd);
  NC_LAUNCH_CHECK();
  return 0;
}

}  // namespace nc
