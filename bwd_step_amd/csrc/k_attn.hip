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
// score accumulator converted to bf16; V^T comes from an LDS tile that is
// transposed in registers while it is staged.  The key order inside one MFMA
// reduction step is permuted identically in both operands, which leaves the
// sum unchanged.
//
// Forward: 128 queries per workgroup (4 wavefronts x 32), 64-key blocks,
// online softmax in the exp2 domain; lse is saved.  Backward: dK/dV kernel
// with 128 keys per workgroup looping over 64-query blocks (P recomputed from
// lse), and a separate dQ kernel with 128 queries per workgroup looping over
// 64-key blocks; no floating-point atomics, so results are reproducible.
// Workgroups with the most causal work are launched first.
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

// ------------------------------------------------------------------ forward, head_dim 128
// K and V tiles ([64 keys][128], 16 KB each) are staged with LDS-direct buffer
// loads into two stages (separate LDS objects, so the compiler does not wait
// on the in-flight stage).  K fragments for S^T = K Q^T are 16-byte reads of
// an XOR-swizzled tile (chunk ^= key & 15).  V^T fragments for O^T = V^T P^T
// come straight from the row-major V tile through ds_read_b64_tr_b16, whose
// per-16-lane-group key offset is chosen to follow the key order that the
// score accumulator already has; the V chunks are swizzled by sw_v(key & 3)
// so that these reads are conflict free.  The kernel stays under 256
// registers per lane so that two workgroups (eight wavefronts) share a
// compute unit and one's softmax overlaps the other's MFMAs.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef short v4i16 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ int sw_v(int r) { return 4 * r + 2 * ((r >> 1) & 1); }
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// One 1 KB block (4 key rows of 128) of a [64][128] tile; V tiles use the
// transposed-read swizzle, K tiles the row swizzle.
template <bool VTILE>
__device__ __forceinline__ void kv_dma(rsrc_t rs, long ld, long col0, int key0, int T, bf16* lds, int blk,
                                       int lane) {
  const int row = blk * 4 + (lane >> 4);
  const int pc = lane & 15;
  const int c = VTILE ? (pc ^ sw_v(row & 3)) : (pc ^ (row & 15));
  const int key = key0 + row;
  const uint32_t off = key < T ? (uint32_t)(((long)key * ld + col0 + c * 8) * 2) : kOOB;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(lds + blk * 512), 16, off, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 k_frag(const bf16* Ks, int row, int chunk) {
  return *reinterpret_cast<const bf16x8*>(Ks + row * 128 + ((chunk ^ (row & 15)) << 3));
}

// V^T fragment: hd rows x*32 + (lane & 31), keys kb + {4g .. 4g+3, 8+4g .. 8+4g+3}, g = lane / 32.
__device__ __forceinline__ bf16x8 vt_frag(const bf16* Vs, int x, int kb, int lane) {
  const int gi = lane >> 4, i = lane & 15;
  const int r = i >> 2, q = i & 3;
  const int chunk = (x * 4 + 2 * (gi & 1) + (q >> 1)) ^ sw_v(r);
  const int col = (chunk << 3) + 4 * (q & 1);
  const int k0 = kb + 4 * (gi >> 1) + r;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)(Vs + k0 * 128 + col));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)(Vs + (k0 + 8) * 128 + col));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}


__global__ void __launch_bounds__(256, 2) attn_fwd128(AttnArgs p) {
  constexpr int HD = 128, KS = 8, HB = 4;
  __shared__ __attribute__((aligned(1024))) bf16 K0[64 * HD];
  __shared__ __attribute__((aligned(1024))) bf16 K1[64 * HD];
  __shared__ __attribute__((aligned(1024))) bf16 V0[64 * HD];
  __shared__ __attribute__((aligned(1024))) bf16 V1[64 * HD];

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

  f32x16 oacc[HB];
#pragma unroll
  for (int x = 0; x < HB; ++x) oacc[x] = f32x16{};
  float mx = -INFINITY, lsum = 0.f;
  const float c = p.scale_log2;

  const int q_last = min(T - 1, q0 + 127);
  const int nkv = q_last / 64 + 1;
  const int wq_min = q0 + wv * 32, wq_max = wq_min + 31;

  // stage block 0
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    kv_dma<false>(rk, p.ldk, colk, 0, T, K0, wv * 4 + i, lane);
    kv_dma<true>(rv, p.ldv, colk, 0, T, V0, wv * 4 + i, lane);
  }
  wait_vmem();
  __syncthreads();

  auto block = [&](const bf16* Ks, const bf16* Vs, bf16* Kn, bf16* Vn, int kb) {
    const bool live = kb + 1 < nkv;
    const int knext = (kb + 1) * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kv_dma<false>(rk, p.ldk, colk, live ? knext : T, T, Kn, wv * 4 + i, lane);
      kv_dma<true>(rv, p.ldv, colk, live ? knext : T, T, Vn, wv * 4 + i, lane);
    }
    const int kbase = kb * 64;
    if (kbase <= wq_max) {
      f32x16 sacc[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        sacc[kk] = f32x16{};
#pragma unroll
        for (int s = 0; s < KS; ++s) sacc[kk] = mfma(k_frag(Ks, kk * 32 + li, 2 * s + g), qf[s], sacc[kk]);
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
      float ps = 0.f;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = ex2(fmaf(sacc[kk][r], c, moff));
          sacc[kk][r] = e;
          ps += e;
        }
      lsum += ps;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const bf16x8 pf = pack8(sacc[kk], t);
#pragma unroll
          for (int x = 0; x < HB; ++x) oacc[x] = mfma(vt_frag(Vs, x, kk * 32 + t * 16, lane), pf, oacc[x]);
        }
    }
  };

  int kb = 0;
  for (; kb + 1 < nkv; kb += 2) {
    block(K0, V0, K1, V1, kb);
    wait_vmem();
    __syncthreads();
    block(K1, V1, K0, V0, kb + 1);
    wait_vmem();
    __syncthreads();
  }
  if (kb < nkv) block(K0, V0, K1, V1, kb);
  wait_vmem();  // the tail's no-op loads still target LDS

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

// ------------------------------------------------------------------ backward, head_dim 128
// Tiles of 64 rows x 128 that are read both ways -- 16-byte row fragments
// (the A operand of S = Q K^T, dP = dO V^T and their transposes) and
// transposed fragments through ds_read_b64_tr_b16 (the A operand of
// dQ^T = K^T dS^T, dK^T = Q^T dS, dV^T = dO^T P) -- use one XOR swizzle of
// the 16-byte chunk index, sw2(row), that is conflict free for both access
// patterns (any 16 aligned rows see 16 distinct chunk slots; within every
// aligned group of 4 rows bits 2-3 differ and bits 1-2 differ).
__device__ __forceinline__ int sw2(int row) { return 4 * (row & 3) + (((row >> 2) & 3) ^ (2 * ((row >> 1) & 1))); }

__device__ __forceinline__ void tile_dma(rsrc_t rs, long ld, long col0, int row0, int T, bf16* lds, int blk,
                                         int lane) {
  const int row = blk * 4 + (lane >> 4);
  const int c = (lane & 15) ^ sw2(row);
  const int t = row0 + row;
  const uint32_t off = t < T ? (uint32_t)(((long)t * ld + col0 + c * 8) * 2) : kOOB;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(lds + blk * 512), 16, off, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 row_frag(const bf16* S, int row, int chunk) {
  return *reinterpret_cast<const bf16x8*>(S + row * 128 + ((chunk ^ sw2(row)) << 3));
}

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

// dQ: 128 queries per workgroup, 32 per wavefront (its qh and dO fragments
// in registers).  Blocks of 64 keys (K and V tiles, 64 rows x 256 bytes with
// the sw2 chunk swizzle) stream through four LDS stages, loaded two blocks
// ahead (same scheme as the dK/dV kernel below).  A block is processed as two
// halves of 32 keys: the dS arithmetic of one half is issued together with
// the S / dP products of the next half, then the dQ products of the half.
__global__ void __launch_bounds__(256, 1) attn_bwd_dq128(AttnArgs p) {
  constexpr int HD = 128, KS = 8, HB = 4;
  constexpr uint32_t kTile = 64 * HD * 2, kStage = 2 * kTile;
  __shared__ __attribute__((aligned(1024))) char smem[4 * kStage];
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  const int T = p.T;
  const int nqb = gridDim.x;
  const int lin = xcd_block(blockIdx.x + nqb * blockIdx.y, nqb * gridDim.y);
  const int qb = nqb - 1 - lin % nqb;  // query blocks of one (b, h) in turn, the longest first
  const int bh = lin / nqb, b = bh / p.H, h = bh % p.H;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, li = lane & 31;
  const int q0 = qb * 128;
  const int qi = q0 + wv * 32 + li;  // this lane's query

  const size_t tok0 = (size_t)b * T;
  const rsrc_t rk = make_rsrc((const bf16*)p.k + tok0 * p.ldk,
                              (uint32_t)(((size_t)(T - 1) * p.ldk + (size_t)(p.H / p.G) * HD) * 2));
  const rsrc_t rv = make_rsrc((const bf16*)p.v + tok0 * p.ldv,
                              (uint32_t)(((size_t)(T - 1) * p.ldv + (size_t)(p.H / p.G) * HD) * 2));
  const long col = (long)(h / p.G) * HD;  // this query head's key/value head
  const int nkv = min(T - 1, q0 + 127) / 64 + 1;  // key blocks up to the diagonal

  uint32_t toff_k[4], toff_v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (wv * 4 + i) * 4 + (lane >> 4);
    const int cc = (lane & 15) ^ sw2(row);
    toff_k[i] = (uint32_t)(((long)row * p.ldk + col + cc * 8) * 2);
    toff_v[i] = (uint32_t)(((long)row * p.ldv + col + cc * 8) * 2);
  }
  // loads of key block j into stage st (8 per wavefront); rows past T and
  // blocks past the last read 0
  auto load_block = [&](int st, int j) {
    const int row0 = j < nkv ? j * 64 : T;
    const uint32_t sb = lds0 + (uint32_t)st * kStage;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = row0 + (wv * 4 + i) * 4 + (lane >> 4) < T;
      dma16(rk, ok ? toff_k[i] + (uint32_t)(row0 * p.ldk * 2) : kOOB, sb + (uint32_t)(wv * 4 + i) * 1024u);
      dma16(rv, ok ? toff_v[i] + (uint32_t)(row0 * p.ldv * 2) : kOOB, sb + kTile + (uint32_t)(wv * 4 + i) * 1024u);
    }
  };
  auto wait_block_and_sync = [&]() { asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory"); };

  load_block(0, 0);
  load_block(1, 1);
  const bf16* qp = (const bf16*)p.q + tok0 * p.ldq + h * HD;
  const bf16* dop = (const bf16*)p.dout + tok0 * p.lddo + h * HD;
  bf16x8 qf[KS], df[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    qf[s] = qi < T ? *reinterpret_cast<const bf16x8*>(qp + (size_t)qi * p.ldq + s * 16 + g * 8) : bf16x8{};
    df[s] = qi < T ? *reinterpret_cast<const bf16x8*>(dop + (size_t)qi * p.lddo + s * 16 + g * 8) : bf16x8{};
  }
  const float nlse = qi < T ? -p.lse[(size_t)bh * T + qi] : 0.f;  // base 2
  // D = rowsum(dO * O) of this lane's query (lanes l and l ^ 32 hold the two
  // halves of the row), also written for the dK/dV kernel that runs next
  float Dl = 0.f;
  {
    const bf16* op = (const bf16*)p.o + tok0 * p.ldo + h * HD;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 o8 = qi < T ? *reinterpret_cast<const bf16x8*>(op + (size_t)qi * p.ldo + s * 16 + g * 8) : bf16x8{};
#pragma unroll
      for (int e = 0; e < 8; ++e) Dl = fmaf(to_f32(df[s][e]), to_f32(o8[e]), Dl);
    }
    Dl += __shfl_xor(Dl, 32, 64);
    if (g == 0 && qi < T) p.Dbuf[(size_t)bh * T + qi] = Dl;
  }
  const float c = p.scale_log2;
  // dP^T accumulators start at -D (one value per lane: its query), so they
  // end at dP - D and dS = P (dP - D) takes one multiply
  f32x16 negD;
#pragma unroll
  for (int r = 0; r < 16; ++r) negD[r] = -Dl;
  f32x16 dq[HB];
#pragma unroll
  for (int x = 0; x < HB; ++x) dq[x] = f32x16{};

  // S^T and dP^T of one half (kk: 32 keys) of the block in stage st.  All 16
  // fragment reads are issued in a scheduling region of their own, ahead of
  // the MFMAs: with one wavefront per SIMD, a read placed next to the MFMA
  // that consumes it stalls that MFMA for the whole LDS latency.
  auto phase_a = [&](uint32_t st, int kk, f32x16& S, f32x16& Pd) {
    const char* sb = smem + st * kStage;
    const bf16* Ks = (const bf16*)sb;
    const bf16* Vs = (const bf16*)(sb + kTile);
    bf16x8 fk[KS], fv[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      fk[s] = row_frag(Ks, kk * 32 + li, 2 * s + g);
      fv[s] = row_frag(Vs, kk * 32 + li, 2 * s + g);
    }
    __builtin_amdgcn_sched_barrier(0);
    S = f32x16{};
    Pd = negD;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      S = mfma(fk[s], qf[s], S);
      Pd = mfma(fv[s], df[s], Pd);
    }
  };
  // dS^T = P (dP - D) of one half as bf16 B operands; MASKED: causal / length mask
  auto phase_b = [&](auto masked, const f32x16& S, const f32x16& Pd, int kh, bf16x8* sf) {
    constexpr bool MASKED = decltype(masked)::value;
    f32x16 dS;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float pr = ex2(fmaf(S[r], c, nlse));
      if constexpr (MASKED) {
        const int key = kh + acc_row(r, g);
        pr = (key > qi || key >= T) ? 0.f : pr;
      }
      dS[r] = pr * Pd[r];
    }
    sf[0] = pack8(dS, 0);
    sf[1] = pack8(dS, 1);
  };
  // dQ += dS K for one half of the block in stage st
  auto phase_c = [&](uint32_t st, int kk, const bf16x8* sf) {
    const bf16* Ks = (const bf16*)(smem + st * kStage);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int x = 0; x < HB; ++x) dq[x] = mfma(tr_frag(Ks, x, kk * 32 + t * 16, lane), sf[t], dq[x]);
  };
  // Instruction interleave of one section: LEAD LDS reads first, then NM
  // groups of one MFMA, NDS LDS reads (for later MFMAs) and NVALU vector
  // instructions.  The lead keeps the fragment reads several MFMAs ahead of
  // their use, so with one wavefront per SIMD an MFMA does not wait out the
  // LDS latency of its own operand.
  auto interleave = [&](auto nm, auto lead, auto nds, auto nvalu) {
    if constexpr (decltype(lead)::value > 0) __builtin_amdgcn_sched_group_barrier(0x100, decltype(lead)::value, 0);
#pragma unroll
    for (int i = 0; i < decltype(nm)::value; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if constexpr (decltype(nds)::value > 0) __builtin_amdgcn_sched_group_barrier(0x100, decltype(nds)::value, 0);
      if constexpr (decltype(nvalu)::value > 0) __builtin_amdgcn_sched_group_barrier(0x002, decltype(nvalu)::value, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  using I0 = std::integral_constant<int, 0>;
  using I2 = std::integral_constant<int, 2>;
  using I6 = std::integral_constant<int, 6>;
  using I8 = std::integral_constant<int, 8>;
  using I16 = std::integral_constant<int, 16>;

  f32x16 Sa, Pa;  // the pending half: S^T and dP^T done, arithmetic not yet
  auto pass = [&](auto masked, int j) {
    const uint32_t cur = (uint32_t)j & 3u, nxt = (uint32_t)(j + 1) & 3u;
    load_block((j + 2) & 3, j + 2);
    const int kbase = j * 64;
    bf16x8 sf[2];
    f32x16 Sb, Pb;
    __builtin_amdgcn_sched_barrier(0);
    phase_a(cur, 1, Sb, Pb);
    phase_b(masked, Sa, Pa, kbase, sf);
    interleave(I16{}, I0{}, I0{}, I6{});
    phase_c(cur, 0, sf);
    interleave(I8{}, I6{}, I2{}, I0{});
    wait_block_and_sync();  // block j + 1
    phase_a(nxt, 0, Sa, Pa);
    phase_b(masked, Sb, Pb, kbase + 32, sf);
    interleave(I16{}, I0{}, I0{}, I6{});
    phase_c(cur, 1, sf);
    interleave(I8{}, I6{}, I2{}, I0{});
  };

  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");  // blocks 0 and 1, qh and dO
  phase_a(0, 0, Sa, Pa);
  // The last two blocks meet the diagonal and a block j with (j + 1) * 64 > T
  // (j >= T / 64) meets the end, so the masked passes are a suffix.  Two
  // loops with one pass body each keep the accumulators in one place (one
  // loop with both bodies behind a branch moved dQ between register files
  // on every trip).
  const int jm = max(0, min(nkv - 2, T / 64));
  int j = 0;
  for (; j < jm; ++j) pass(std::false_type{}, j);
  for (; j < nkv; ++j) pass(std::true_type{}, j);
  wait_vmem();  // the loads of the two blocks past the end still target LDS

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

// dK, dV: 128 keys per workgroup, 32 per wavefront (its K and -V fragments in
// registers).  Blocks of 64 queries (qh, dO and their lse and D) stream
// through four LDS stages, loaded two blocks ahead.  A block is processed as
// two halves of 32 queries, software-pipelined: the P / dS arithmetic of one
// half is issued together with the S / dP products of the next half, then
// the dV / dK products of the half follow.  With -V in place of V the dP
// accumulator starts at D and ends at D - dP, so P (D - dP) = -dS comes out
// of one multiply; the sign is restored when dK is written.
//
// LDS: one array of four 36-KB stages (qh tile, dO tile: 64 rows x 256 bytes
// with the sw2 chunk swizzle; then four 1-KB vector slots: lse (base 2), D,
// and copies of both, one slot loaded by each wavefront).
__global__ void __launch_bounds__(256, 1) attn_bwd_dkdv128(AttnArgs p) {
  constexpr int HD = 128, KS = 8, HB = 4;
  constexpr uint32_t kTile = 64 * HD * 2, kStage = 2 * kTile + 4096;
  __shared__ __attribute__((aligned(1024))) char smem[4 * kStage];
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  const int T = p.T;
  const int nkb = gridDim.x;
  const int lin = xcd_block(blockIdx.x + nkb * blockIdx.y, nkb * gridDim.y);
  const int kbk = lin % nkb;  // key blocks of one (b, h) in turn, the longest first
  const int bh = lin / nkb, b = bh / p.H, h = bh % p.H;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, li = lane & 31;
  const int k0 = kbk * 128;
  const int wk = k0 + wv * 32;  // the wavefront's first key
  const int kj = wk + li;       // this lane's key
  const size_t tok0 = (size_t)b * T;
  const rsrc_t rq = make_rsrc((const bf16*)p.q + tok0 * p.ldq,
                              (uint32_t)(((size_t)(T - 1) * p.ldq + (size_t)p.H * HD) * 2));
  const rsrc_t ro = make_rsrc((const bf16*)p.dout + tok0 * p.lddo,
                              (uint32_t)(((size_t)(T - 1) * p.lddo + (size_t)p.H * HD) * 2));
  // wavefronts 0 and 2 load lse (base 2), 1 and 3 load D
  const rsrc_t rv = make_rsrc((wv & 1) ? (const void*)(p.Dbuf + (size_t)bh * T) : (const void*)(p.lse + (size_t)bh * T),
                              (uint32_t)T * 4u);
  const long col = (long)h * HD;
  const int qb0 = k0 / 64;
  const int nb = (T + 63) / 64 - qb0;  // query blocks at or after the diagonal

  // Per-lane byte offsets of this wavefront's tile loads (4 slots of 4 rows
  // for each tile) relative to the block's first row, and of its vector load.
  uint32_t toff_q[4], toff_o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (wv * 4 + i) * 4 + (lane >> 4);
    const int cc = (lane & 15) ^ sw2(row);
    toff_q[i] = (uint32_t)(((long)row * p.ldq + col + cc * 8) * 2);
    toff_o[i] = (uint32_t)(((long)row * p.lddo + col + cc * 8) * 2);
  }
  // loads of query block j into stage st (9 per wavefront); rows past T and
  // blocks past the last read 0
  auto load_block = [&](int st, int j) {
    const int row0 = j < nb ? (qb0 + j) * 64 : T;
    const uint32_t sb = lds0 + (uint32_t)st * kStage;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = row0 + (wv * 4 + i) * 4 + (lane >> 4);
      const bool ok = row < T;
      dma16(rq, ok ? toff_q[i] + (uint32_t)(row0 * p.ldq * 2) : kOOB, sb + (uint32_t)(wv * 4 + i) * 1024u);
      dma16(ro, ok ? toff_o[i] + (uint32_t)(row0 * p.lddo * 2) : kOOB, sb + kTile + (uint32_t)(wv * 4 + i) * 1024u);
    }
    const int t = row0 + 4 * lane;
    dma16(rv, (lane < 16 && t < T) ? (uint32_t)t * 4u : kOOB, sb + 2 * kTile + (uint32_t)wv * 1024u);
  };
  // Loads retire in issue order: with the 9 loads of the newest block still
  // in flight, the previous block has landed.  The barrier publishes it and
  // orders every wavefront's reads of older stages before the next loads.
  auto wait_block_and_sync = [&]() { asm volatile("s_waitcnt vmcnt(9)\n\ts_barrier" ::: "memory"); };

  load_block(0, 0);
  load_block(1, 1);
  const bf16* kp = (const bf16*)p.k + tok0 * p.ldk + (h / p.G) * HD;
  const bf16* vp = (const bf16*)p.v + tok0 * p.ldv + (h / p.G) * HD;
  bf16x8 kf[KS], vn[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    kf[s] = kj < T ? *reinterpret_cast<const bf16x8*>(kp + (size_t)kj * p.ldk + s * 16 + g * 8) : bf16x8{};
    const bf16x8 v = kj < T ? *reinterpret_cast<const bf16x8*>(vp + (size_t)kj * p.ldv + s * 16 + g * 8) : bf16x8{};
    vn[s] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, v) ^ 0x80008000u);  // -V
  }
  f32x16 dk[HB], dv[HB];
#pragma unroll
  for (int x = 0; x < HB; ++x) { dk[x] = f32x16{}; dv[x] = f32x16{}; }
  const float c = p.scale_log2;

  // S and D - dP of one half (mi) of the block in stage st.  The fragment and
  // D reads are issued in a scheduling region of their own, ahead of the
  // MFMAs, so that no MFMA waits out the LDS latency of its own operand.
  auto phase_a = [&](uint32_t st, int mi, f32x16& S, f32x16& Pd) {
    const char* sb = smem + st * kStage;
    const bf16* Qs = (const bf16*)sb;
    const bf16* Os = (const bf16*)(sb + kTile);
    const float* Ds = (const float*)(sb + 2 * kTile) + 256;
    bf16x8 fq[KS], fo[KS];
    f32x4 d4[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) d4[rb] = *reinterpret_cast<const f32x4*>(Ds + mi * 32 + 8 * rb + 4 * g);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      fq[s] = row_frag(Qs, mi * 32 + li, 2 * s + g);
      fo[s] = row_frag(Os, mi * 32 + li, 2 * s + g);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      // accumulator registers 4 rb .. 4 rb + 3 hold four consecutive queries
      Pd[4 * rb + 0] = d4[rb].x;
      Pd[4 * rb + 1] = d4[rb].y;
      Pd[4 * rb + 2] = d4[rb].z;
      Pd[4 * rb + 3] = d4[rb].w;
    }
    S = f32x16{};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      S = mfma(fq[s], kf[s], S);
      Pd = mfma(fo[s], vn[s], Pd);
    }
  };
  // P = exp2(S c - lse) and -dS = P (D - dP) of one half, as bf16 B operands;
  // MASKED: apply the causal / length mask (passes that meet the diagonal or T)
  auto phase_b = [&](auto masked, const f32x16& S, const f32x16& Pd, uint32_t st, int mi, int qh, bf16x8* pf,
                     bf16x8* sf) {
    constexpr bool MASKED = decltype(masked)::value;
    const float* Ls = (const float*)(smem + st * kStage + 2 * kTile);
    f32x16 P, dS;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(Ls + mi * 32 + 8 * rb + 4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * rb + e;
        float pr = ex2(fmaf(S[r], c, -l4[e]));
        if constexpr (MASKED) {
          const int q = qh + 8 * rb + 4 * g + e;
          pr = (q < kj || q >= T) ? 0.f : pr;
        }
        P[r] = pr;
        dS[r] = pr * Pd[r];
      }
    }
    pf[0] = pack8(P, 0);
    pf[1] = pack8(P, 1);
    sf[0] = pack8(dS, 0);
    sf[1] = pack8(dS, 1);
  };
  // dV += P^T dO and dK' += (-dS)^T qh for one half of the block in stage st
  auto phase_c = [&](uint32_t st, int mi, const bf16x8* pf, const bf16x8* sf) {
    const char* sb = smem + st * kStage;
    const bf16* Qs = (const bf16*)sb;
    const bf16* Os = (const bf16*)(sb + kTile);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int x = 0; x < HB; ++x) {
        dv[x] = mfma(tr_frag(Os, x, mi * 32 + t * 16, lane), pf[t], dv[x]);
        dk[x] = mfma(tr_frag(Qs, x, mi * 32 + t * 16, lane), sf[t], dk[x]);
      }
  };
  // Instruction interleave of one pipelined section of 16 MFMAs: LEAD LDS
  // reads first, then per MFMA NDS LDS reads (for later MFMAs) and NVALU
  // vector instructions, so that the reads run ahead of their MFMAs.
  auto interleave = [&](auto lead, auto nds, auto nvalu) {
    if constexpr (decltype(lead)::value > 0) __builtin_amdgcn_sched_group_barrier(0x100, decltype(lead)::value, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if constexpr (decltype(nds)::value > 0) __builtin_amdgcn_sched_group_barrier(0x100, decltype(nds)::value, 0);
      if constexpr (decltype(nvalu)::value > 0) __builtin_amdgcn_sched_group_barrier(0x002, decltype(nvalu)::value, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  using I0 = std::integral_constant<int, 0>;
  using I2 = std::integral_constant<int, 2>;
  using I4 = std::integral_constant<int, 4>;
  using I6 = std::integral_constant<int, 6>;
  using I8 = std::integral_constant<int, 8>;

  // One pass over block j (in stage j mod 4): its second half, then the first
  // half of block j + 1, whose loads are waited for in the middle.
  f32x16 Sa, Pa;  // the pending half: S and D - dP, products done, arithmetic not yet
  auto pass = [&](auto masked, int j) {
    const uint32_t cur = (uint32_t)j & 3u, nxt = (uint32_t)(j + 1) & 3u;
    load_block((j + 2) & 3, j + 2);
    const int qbase = (qb0 + j) * 64;
    bf16x8 pf[2], sf[2];
    f32x16 Sb, Pb;
    __builtin_amdgcn_sched_barrier(0);
    phase_a(cur, 1, Sb, Pb);
    phase_b(masked, Sa, Pa, cur, 0, qbase, pf, sf);
    interleave(I4{}, I0{}, I6{});
    phase_c(cur, 0, pf, sf);
    interleave(I8{}, I2{}, I0{});
    wait_block_and_sync();  // block j + 1
    phase_a(nxt, 0, Sa, Pa);
    phase_b(masked, Sb, Pb, cur, 1, qbase + 32, pf, sf);
    interleave(I4{}, I0{}, I6{});
    phase_c(cur, 1, pf, sf);
    interleave(I8{}, I2{}, I0{});
  };

  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");  // blocks 0 and 1, K and V
  phase_a(0, 0, Sa, Pa);
  // The first two blocks meet the diagonal and a block j with
  // (qb0 + j + 1) * 64 > T (j >= T / 64 - qb0) meets the end: masked passes
  // are a prefix and a suffix, each range run by a loop of its own so that
  // the accumulators stay in one register file.
  const int j_end = min(nb, max(2, T / 64 - qb0));
  int j = 0;
  for (; j < min(2, nb); ++j) pass(std::true_type{}, j);
  for (; j < j_end; ++j) pass(std::false_type{}, j);
  for (; j < nb; ++j) pass(std::true_type{}, j);
  wait_vmem();  // the loads of the two blocks past the end still target LDS

  if (kj >= T) return;
  const float sc = -p.scale;  // dK' = -dK
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
      // the dQ kernel computes D = rowsum(dO * O) for the dK/dV kernel
      attn_bwd_dq128<<<gq, 256, 0, s>>>(p);
      attn_bwd_dkdv128<<<gk, 256, 0, s>>>(p);
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
