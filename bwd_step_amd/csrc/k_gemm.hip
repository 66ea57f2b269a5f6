// Matrix products for every linear layer of the model:
//   C[i, j] = sum_k A(i, k) * B(j, k)
// forward y = x W^T (both operands k-contiguous), input gradient dx = dy W
// (B is W stored [k][j]) and weight gradient dW = dy^T x (both operands
// stored [k][i]); see "nanochat explainer", Modern architecture choices, for
// the layers (QKV and output projections, ReLU² MLP, untied LM head).
//
// bf16 path: v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  A 256-thread
// workgroup owns a 256x256 output tile; its four wavefronts each own 128x128
// (4x4 MFMA blocks of 32x32).  The grid is persistent (one workgroup per
// compute unit walking (tile, K split) items).  K advances through four LDS
// stages of 32-deep slices filled by LDS-direct buffer loads issued three
// slices ahead.  k-contiguous slices hold 64-byte rows with an XOR-swizzled
// 16-byte chunk index; operands whose reduction index is strided are staged
// as they lie in memory (k rows of 256 m) and read transposed with
// ds_read_b64_tr_b16.  Both layouts are read without bank conflicts.
// Products whose operands are both k-contiguous (the forward products and
// the LM-head logits) run 64-deep pairs instead, through a ring of five
// 32 KB slots (160 KB), so that their rows load as 128-byte segments.
//
// fp32 debug path: a plain 64x64 LDS-tiled SIMT kernel with the same epilogues.
//
// Epilogues are fused so that each output is written once: fp32 store or
// accumulate, bf16 store, residual add into the fp32 stream, ReLU² (stores
// g = max(u,0)^2 only), and the ReLU² backward (du = dg * 2 sqrt(g)).
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace nc {

struct GemmParams {
  const void* A;
  const void* B;
  long lda, ldb;
  uint32_t a_bytes, b_bytes;  // extent of each operand (buffer bound; beyond it loads read 0)
  int M, N, K;
  int kchunk;  // K range per split (multiple of 128 when split)
  int splits;
  int tiles_m, tiles_n;
  int group;  // tile-rows per group of the tile walk
  int batch;  // independent products (1 unless batched)
  int sym;    // symmetric square result: only tiles tm <= tn, each also stored transposed
  long a_bs, b_bs;  // bytes between consecutive batch members' A and B
  EpiArgs e;
};

// ------------------------------------------------------------------ epilogue
// Four consecutive columns j .. j+3 of row i (N is a multiple of 4, so the
// group is either wholly inside or wholly outside the matrix).
template <class T>
__device__ __forceinline__ void store4(T* p, f32x4 v) {
  if constexpr (sizeof(T) == 2) {
    u32x2 w;
    w.x = pack_bf16x2(v.x, v.y);
    w.y = pack_bf16x2(v.z, v.w);
    *reinterpret_cast<u32x2*>(p) = w;
  } else {
    *reinterpret_cast<f32x4*>(p) = v;
  }
}
template <class T>
__device__ __forceinline__ f32x4 load4(const T* p) {
  if constexpr (sizeof(T) == 2) {
    const u32x2 w = *reinterpret_cast<const u32x2*>(p);
    return f32x4{bf16lo_to_f32(w.x), bf16hi_to_f32(w.x), bf16lo_to_f32(w.y), bf16hi_to_f32(w.y)};
  } else {
    return *reinterpret_cast<const f32x4*>(p);
  }
}

// ReLU² backward from the saved g = relu(u)^2: d/du relu(u)^2 = 2 relu(u) =
// 2 sqrt(g), so u itself is never stored.  g >= 0 comes from bf16 storage and
// the result is rounded to bf16, so the hardware square root (v_sqrt_f32,
// 1 ulp) replaces the correctly rounded expansion, which costs about ten
// VALU instructions per element in an MFMA epilogue.
__device__ __forceinline__ f32x4 drelu2(f32x4 dg, f32x4 g) {
  return f32x4{2.f * __builtin_amdgcn_sqrtf(g.x) * dg.x, 2.f * __builtin_amdgcn_sqrtf(g.y) * dg.y,
               2.f * __builtin_amdgcn_sqrtf(g.z) * dg.z, 2.f * __builtin_amdgcn_sqrtf(g.w) * dg.w};
}

template <int EPI, class T = bf16>
__device__ __forceinline__ void epi_apply4(const EpiArgs& e, int split, long i, long j, f32x4 v) {
  if constexpr (EPI == EPI_F32 || EPI == EPI_F32_ACC) {
    f32x4* c = reinterpret_cast<f32x4*>(e.c32 + (size_t)split * e.split_stride + i * e.ldc + j);
    if constexpr (EPI == EPI_F32_ACC) v += *c;
    *c = v;
  } else if constexpr (EPI == EPI_RESID) {
    f32x4* c = reinterpret_cast<f32x4*>(e.c32 + i * e.ldc + j);
    *c = *c + v;
  } else if constexpr (EPI == EPI_LP) {
    store4((T*)e.c_lp + i * e.ld_lp + j, v);
  } else if constexpr (EPI == EPI_RELU2) {
    const f32x4 r{fmaxf(v.x, 0.f), fmaxf(v.y, 0.f), fmaxf(v.z, 0.f), fmaxf(v.w, 0.f)};
    store4((T*)e.c_lp + i * e.ld_lp + j, r * r);
  } else if constexpr (EPI == EPI_DRELU2) {
    store4((T*)e.c_lp + i * e.ld_lp + j, drelu2(v, load4((const T*)e.aux + i * e.ld_aux + j)));
  } else if constexpr (EPI == EPI_AXPBY) {
    const f32x4 x = load4((const T*)e.aux + i * e.ld_aux + j);
    store4((T*)e.c_lp + i * e.ld_lp + j,
           f32x4{fmaf(e.alpha, x.x, e.beta_f * v.x), fmaf(e.alpha, x.y, e.beta_f * v.y),
                 fmaf(e.alpha, x.z, e.beta_f * v.z), fmaf(e.alpha, x.w, e.beta_f * v.w)});
  }
}

template <int EPI, class T>
__device__ __forceinline__ void epi_apply(const EpiArgs& e, int split, long i, long j, float v) {
  if constexpr (EPI == EPI_F32) {
    float* c = e.c32 + (size_t)split * e.split_stride + i * e.ldc + j;
    if (e.beta) *c += v; else *c = v;
  } else if constexpr (EPI == EPI_RESID) {
    e.c32[i * e.ldc + j] += v;
  } else if constexpr (EPI == EPI_LP) {
    ((T*)e.c_lp)[i * e.ld_lp + j] = from_f32<T>(v);
  } else if constexpr (EPI == EPI_RELU2) {
    const float r = v > 0.f ? v : 0.f;
    ((T*)e.c_lp)[i * e.ld_lp + j] = from_f32<T>(r * r);
  } else if constexpr (EPI == EPI_DRELU2) {
    const float g = to_f32(((const T*)e.aux)[i * e.ld_aux + j]);
    ((T*)e.c_lp)[i * e.ld_lp + j] = from_f32<T>(2.f * sqrtf(g) * v);
  } else if constexpr (EPI == EPI_AXPBY) {
    const float x = to_f32(((const T*)e.aux)[i * e.ld_aux + j]);
    ((T*)e.c_lp)[i * e.ld_lp + j] = from_f32<T>(fmaf(e.alpha, x, e.beta_f * v));
  }
}

// ------------------------------------------------------------------ MFMA path
constexpr int kBK = 32;  // K depth of one staged slice
constexpr uint32_t kOOB = 0x80000000u;  // buffer offset past every operand: loads return 0

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef short v4i16 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// k-contiguous slices are [256 rows][32 k] (64-byte rows of four 16-byte
// chunks); the chunk index is XOR-ed with (row >> 2) & 3.  A 16-byte LDS read
// of a wavefront is served in four 16-lane phases over 64 four-byte banks
// (measured on gfx950): a phase is the four lane quads 4q .. 4q+3 of one
// 32-lane half whose quad index q has the same bit parity.  A fragment read
// puts 32 consecutive rows on the lanes of a half, so the four quads of a
// phase have distinct q mod 4 = (row >> 2) & 3, and the four rows of a quad
// lie in distinct 64-byte quarters of the 256-byte bank window: the swizzled
// chunks fill all 16 slots.
__device__ __forceinline__ int swf(int row) { return (row >> 2) & 3; }
__device__ __forceinline__ int swz(int row, int kc) { return row * kBK + ((kc ^ swf(row)) << 3); }

// m-contiguous slices are [32 k][256 m]; the 16-byte chunk index is XOR-ed
// with this function of (k & 3): the four k-rows of one transposed read land
// in four different 64-byte quarters of a 256-byte bank window (bits 2-3)
// and, pairwise, in different halves of a 128-byte window (bits 1-2).
__device__ __forceinline__ int swk(int k) { const int r = k & 3; return 4 * r + 2 * ((r >> 1) & 1); }

// Loads of a 32-deep slice of a 256-row operand: 16 blocks of 1 KB, one
// wavefront LDS-direct buffer load (64 lanes x 16 B) each, into consecutive
// LDS slots; each lane picks the global chunk that belongs at its slot.  The
// per-lane byte offset of block b relative to the slice's first k is fixed
// for a work item (computed once); the slice itself is selected by moving the
// buffer's base address (scalar work), and a slice past the item's K range
// gets a zero-length buffer, so every one of its loads reads 0.  Rows past
// the operand (m >= M) get an offset past any buffer.
template <bool KMAJ>
__device__ __forceinline__ uint32_t dma_voff(long ld, int row0, int rows_lim, int b, int lane) {
  if constexpr (KMAJ) {
    const int row = b * 16 + (lane >> 2);
    const int kc = (lane & 3) ^ swf(row);
    const int gr = row0 + row;
    return gr < rows_lim ? (uint32_t)(((long)gr * ld + kc * 8) * 2) : kOOB;
  } else {
    const int k = 2 * b + (lane >> 5);
    const int mc = (lane & 31) ^ swk(k);
    const int gm = row0 + mc * 8;
    return gm < rows_lim ? (uint32_t)(((long)k * ld + gm) * 2) : kOOB;
  }
}
// The k offset within the slice of the chunk a lane loads in block b
// (k-contiguous operands only; used to cut a final partial slice).
__device__ __forceinline__ int dma_kofs(int b, int lane) {
  const int row = b * 16 + (lane >> 2);
  return ((lane & 3) ^ swf(row)) * 8;
}
// AUX: cache-policy bits of the load.  sc0 (1) measured +18% on products
// whose operands are both k-strided (the weight gradients, long K), -2..5%
// on the others, so only those set it.
template <int AUX>
__device__ __forceinline__ void dma_issue(rsrc_t rs, uint32_t voff, bf16* lds, int b) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(lds + b * 512), 16, voff, 0, 0, AUX);
}

__device__ __forceinline__ v4i16 tr16(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)p);
}

// MFMA 32x32x16 operand fragment for tile rows rb..rb+31 and k-step s (0, 1):
// lane l holds row rb + (l & 31) and k = 16 s + 8 (l >> 5) + 0..7.
template <bool KMAJ>
__device__ __forceinline__ bf16x8 read_frag(const bf16* lds, int rb, int s, int lane) {
  if constexpr (KMAJ) {
    return *reinterpret_cast<const bf16x8*>(lds + swz(rb + (lane & 31), 2 * s + (lane >> 5)));
  } else {
    // ds_read_b64_tr_b16: in each 16-lane group, lane j receives element j % 4
    // of the 8-byte blocks addressed by lanes 4r + j/4 (r = 0..3).  Lane
    // 4r + q addresses row k0 + r, columns m0 + 4q .. m0 + 4q + 3, so lane j
    // gets (k0 + r, m0 + j) for r = 0..3; two reads give the 8 k values.
    const int gi = lane >> 4, i = lane & 15;
    const int m0 = rb + 16 * (gi & 1);
    const int kb = 16 * s + 8 * (gi >> 1);
    const int r = i >> 2, q = i & 3;
    const int cm = ((m0 >> 3) + (q >> 1)) ^ swk(r);  // (kb + r) & 3 == r
    const int col = (cm << 3) + 4 * (q & 1);
    const v4i16 lo = tr16(lds + (kb + r) * 256 + col);
    const v4i16 hi = tr16(lds + (kb + 4 + r) * 256 + col);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Vector memory operations retire in issue order.  Loads run three slices
// ahead and each slice is issued as two halves of 4 loads per wavefront, one
// per MFMA step.  In the middle of slice s the loads still allowed in flight
// are those of slice s+2 and the first half of s+3 (12); after them slice s+1
// has landed in LDS, and the barrier publishes it to the whole workgroup
// (a __syncthreads() would also wait for the younger slices).  lgkmcnt(0):
// this wavefront's reads of slice s are complete, so after the barrier the
// loads that follow may overwrite the stage of slice s-1 (stage (s+3) mod 4).
__device__ __forceinline__ void wait_next_slice_and_sync() {
  asm volatile("s_waitcnt vmcnt(12) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// Prologue: three slices (24 loads) issued, slice 0 needed.
__device__ __forceinline__ void wait_first_slice_and_sync() {
  asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
}

// ---- 64-deep pairs (P64), for products whose operands are both
// k-contiguous.  K advances in pairs of 64-deep slices; a pair is loaded as
// two 32 KB halves, the A half ([256 rows][64 k]) and the B half, with
// 128-byte rows (half the L2 requests of the 64-byte rows of a 32-deep
// slice; measured 46.5 against 30 B/clk per CU from L2) whose 16-byte chunk
// index is XOR-ed with (row >> 1) & 7: the 16 lanes of a read phase (see
// swf) cover rows r with the same r & 1 in pairs of 8 distinct
// (r >> 1) & 7, so their chunks fill all 16 slots.  Wavefront wv loads
// blocks b = wv + 4 q (q = 0..7) of 1 KB, rows 8 b + lane / 8; the swizzle
// of block b depends on b only through b & 1 = wv & 1, so one per-lane
// offset serves all eight and block b adds the scalar b * 16 ld bytes.
// The buffer range check covers the per-lane offset only, not that scalar
// part, so no row of a pair-loop tile may lie past the operand: a tile that
// would cross the end of M (or N) is moved back to end at the last row
// (the operands have at least 256 rows), and its epilogue writes only the
// rows (columns) from the unmoved tile start on, which no other tile owns.
__device__ __forceinline__ uint32_t pair_voff(long ld, int row0, int wv, int lane) {
  const int kc = (lane & 7) ^ ((4 * (wv & 1) + (lane >> 4)) & 7);
  return (uint32_t)((((long)row0 + (lane >> 3)) * ld + kc * 8) * 2);
}
// LDS-direct load written as inline assembly: 64 lanes x 16 bytes from the
// buffer (per-lane offset voff plus the scalar soff) into the 1 KB at LDS byte
// address lds.  The compiler does not see it, so it adds no waits for it; the
// loop counts these loads and waits itself.  No memory clobber: the loads
// write slots that no read in flight touches, and the reads of a slot come
// after the barrier asm (which has one) that follows its wait.  m0 (the LDS
// destination) is saved and restored.
__device__ __forceinline__ void dma_lds(rsrc_t rs, uint32_t voff, uint32_t soff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(rs), "s"(soff));
}
// KTAIL: a k-contiguous operand has K % 32 != 0, so the last slice of the
// last K split is cut per lane (a k-strided operand ends with its buffer).
// BAT: batched / symmetric products (p.batch, p.sym); without it those fields
// are ignored and the hot-path instantiations carry none of their logic.
// P64: the main loop runs 64-deep pairs through a ring of five 32 KB slots
// (both operands k-contiguous, K a multiple of 64, neither KTAIL nor BAT).
template <bool AK, bool BKM, int EPI, bool KTAIL, bool BAT, bool P64>
__global__ void __launch_bounds__(256, 1) gemm_mfma_kernel(GemmParams p) {
  static_assert(!P64 || (AK && BKM && !KTAIL && !BAT), "pair loop: k-contiguous operands only");
  constexpr int BM = 256, BN = 256, WM = 2, WN = 2;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  // Persistent: workgroup w owns work items (tile, K split) w', w' + G, ...
  // (G = grid size).  Workgroup ids are dealt round-robin to the 8 XCDs, so
  // w' gives every XCD a contiguous run of logical items per round; tiles are
  // walked in column groups of 8 tile-rows so that neighbours share A rows and
  // B columns in the XCD's L2.
  const int G = gridDim.x;
  const int ntiles = (BAT && p.sym) ? p.tiles_m * (p.tiles_m + 1) / 2 : p.tiles_m * p.tiles_n;
  const int per_batch = ntiles * p.splits;
  const int nitems = BAT ? per_batch * p.batch : per_batch;
  const int wfirst = (G & 7) == 0 ? (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3) : blockIdx.x;
  if (wfirst >= nitems) return;

  struct Item {
    int m0, n0, kbeg, kend, nk, split, b;
    int mlo, nlo;  // first row / column the epilogue writes (m0, n0 unless the tile was moved back)
    bool mir;  // off-diagonal tile of a symmetric result: also stored transposed
  };
  auto item = [&](int i) {
    Item r;
    if constexpr (BAT) {
      r.b = i / per_batch;
      i -= r.b * per_batch;
    } else {
      r.b = 0;
    }
    r.split = i / ntiles;
    int t = i - r.split * ntiles;
    if (BAT && p.sym) {
      // upper triangle, row by row: tile-row tm holds tiles_m - tm tiles
      int tm = 0;
      while (t >= p.tiles_m - tm) {
        t -= p.tiles_m - tm;
        ++tm;
      }
      r.m0 = tm * BM;
      r.n0 = (tm + t) * BN;
      r.mir = t != 0;
    } else {
      const int group_span = p.group * p.tiles_n;
      const int first_m = (t / group_span) * p.group;
      const int gsize = min(p.tiles_m - first_m, p.group);
      r.m0 = (first_m + (t % group_span) % gsize) * BM;
      r.n0 = ((t % group_span) / gsize) * BN;
      r.mir = false;
    }
    r.mlo = r.m0;
    r.nlo = r.n0;
    if constexpr (P64) {
      // the last tile-row / tile-column ends at the operand's last row
      r.m0 = min(r.m0, p.M - BM);
      r.n0 = min(r.n0, p.N - BN);
    }
    r.kbeg = r.split * p.kchunk;
    r.kend = min(p.K, r.kbeg + p.kchunk);
    r.nk = max((r.kend - r.kbeg + kBK - 1) / kBK, 0);
    return r;
  };

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wv / WN, wn = wv % WN;
  // byte step of the buffer base per k
  const long a_kstep = AK ? 2 : p.lda * 2, b_kstep = BKM ? 2 : p.ldb * 2;
  // buffer of the slice starting at k0 (a zero-length one when it is dead)
  auto slice_rsrc = [&](const void* base, uint32_t bytes, long kstep, int k0, bool live) {
    const long sh = live ? (long)k0 * kstep : 0;
    return make_rsrc((const char*)base + sh, live ? bytes - (uint32_t)sh : 0u);
  };
  auto a_base = [&](const Item& it_) {
    return BAT ? (const void*)((const char*)p.A + it_.b * p.a_bs) : p.A;
  };
  auto b_base = [&](const Item& it_) {
    return BAT ? (const void*)((const char*)p.B + it_.b * p.b_bs) : p.B;
  };
  // per-lane offsets of this wavefront's four blocks of A and B for an item
  auto item_voff = [&](const Item& it_, uint32_t* va, uint32_t* vb) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      va[q] = dma_voff<AK>(p.lda, it_.m0, p.M, wv * 4 + q, lane);
      vb[q] = dma_voff<BKM>(p.ldb, it_.n0, p.N, wv * 4 + q, lane);
    }
  };
  // The loads of blocks q0, q0+1 of the slice starting at k0 (ending the K range at kend).
  auto issue2 = [&](bf16* an, bf16* bn, const uint32_t* va, const uint32_t* vb, rsrc_t rsa, rsrc_t rsb, int q0,
                    int k0, int kend) {
#pragma unroll
    for (int q = q0; q < q0 + 2; ++q) {
      uint32_t oa = va[q], ob = vb[q];
      if constexpr (KTAIL) {
        if (AK && k0 + dma_kofs(wv * 4 + q, lane) >= kend) oa = kOOB;
        if (BKM && k0 + dma_kofs(wv * 4 + q, lane) >= kend) ob = kOOB;
      }
      constexpr int kAux = (!AK && !BKM) ? 1 : 0;
      dma_issue<kAux>(rsa, oa, an, wv * 4 + q);
      dma_issue<kAux>(rsb, ob, bn, wv * 4 + q);
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int c = 0; c < FN; ++c) acc[a][c] = f32x16{};

  // Load one whole slice (4 blocks of A and 4 of B per wavefront).
  auto load_slice = [&](bf16* an, bf16* bn, const uint32_t* va, const uint32_t* vb, const Item& it_, int j) {
    const int k0 = it_.kbeg + j * kBK;
    const bool live = j < it_.nk;
    const rsrc_t rsa = slice_rsrc(a_base(it_), p.a_bytes, a_kstep, k0, live);
    const rsrc_t rsb = slice_rsrc(b_base(it_), p.b_bytes, b_kstep, k0, live);
    issue2(an, bn, va, vb, rsa, rsb, 0, k0, it_.kend);
    issue2(an, bn, va, vb, rsa, rsb, 2, k0, it_.kend);
  };

  // Operand fragments: f0 (k 0..15 of a slice) is read one slice ahead, f1
  // (k 16..31) during the slice's first MFMA step.
  bf16x8 fa0[FM], fb0[FN];
  auto read_step = [&](const bf16* as, const bf16* bs, int st, bf16x8* fa, bf16x8* fb) {
#pragma unroll
    for (int a = 0; a < FM; ++a) fa[a] = read_frag<AK>(as, wm * TM + a * 32, st, lane);
#pragma unroll
    for (int c = 0; c < FN; ++c) fb[c] = read_frag<BKM>(bs, wn * TN + c * 32, st, lane);
  };
  // One MFMA step over the wavefront's 4x4 blocks, interleaved (by
  // sched_group_barrier) with the NR LDS fragment reads and the 4 loads
  // issued in the same step, so the matrix cores are not left waiting for
  // their issue.
  constexpr int NR = (AK ? FM : 2 * FM) + (BKM ? FN : 2 * FN);
  auto mfma_step = [&](const bf16x8* fa, const bf16x8* fb) {
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
      for (int c = 0; c < FN; ++c)
        acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[c], fa[a], acc[a][c], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < FM * FN; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if ((i & 7) == 3) __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
    }
    if (NR > FM * FN) __builtin_amdgcn_sched_group_barrier(0x100, NR - FM * FN, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  // One staged 32-deep slice (in as/bs; the next slice is in as_nx/bs_nx) and
  // the loads of slice j of item it_ (into an/bn, with the item's offsets va/vb).
  auto compute = [&](const bf16* as, const bf16* bs, const bf16* as_nx, const bf16* bs_nx, bf16* an, bf16* bn,
                     const uint32_t* va, const uint32_t* vb, const Item& it_, int j, bool alive) {
    const int k0 = it_.kbeg + j * kBK;
    const bool live = alive && j < it_.nk;
    const rsrc_t rsa = slice_rsrc(a_base(it_), p.a_bytes, a_kstep, k0, live);
    const rsrc_t rsb = slice_rsrc(b_base(it_), p.b_bytes, b_kstep, k0, live);
    bf16x8 fa1[FM], fb1[FN];
    issue2(an, bn, va, vb, rsa, rsb, 0, k0, it_.kend);
    read_step(as, bs, 1, fa1, fb1);
    mfma_step(fa0, fb0);
    wait_next_slice_and_sync();
    issue2(an, bn, va, vb, rsa, rsb, 2, k0, it_.kend);
    read_step(as_nx, bs_nx, 0, fa0, fb0);
    mfma_step(fa1, fb1);
  };

  // Transposed copy of four outputs (i, j..j+3) of a symmetric result: C[j+e][i].
  // The 32 lanes of a half-wavefront hold 32 consecutive i, so each of the
  // four stores covers 64 contiguous bytes.
  auto store_mirror = [&](long i, long j, long ib, f32x4 v) {
    bf16* cb = (bf16*)p.e.c_lp;
#pragma unroll
    for (int e = 0; e < 4; ++e) cb[(j + e + ib) * p.e.ld_lp + i] = from_f32<bf16>(v[e]);
  };

  // Epilogue.  The MFMA computed C^T blocks (B fragment as the row operand), so
  // a lane holds output row m = lane & 31 of its block and, in register
  // group q = r / 4, the four consecutive columns 8 q + 4 (lane / 32) + 0..3.
  auto epilogue = [&](const Item& ci) {
#pragma unroll
    for (int a = 0; a < FM; ++a) {
      const long i = ci.m0 + wm * TM + a * 32 + (lane & 31);
#pragma unroll
      for (int c = 0; c < FN; ++c) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const long j = ci.n0 + wn * TN + c * 32 + 8 * q + 4 * (lane >> 5);
          if constexpr (BAT) {
            // batch member b writes rows b M ..; a symmetric result also its mirror tile
            const f32x4 v{acc[a][c][4 * q], acc[a][c][4 * q + 1], acc[a][c][4 * q + 2], acc[a][c][4 * q + 3]};
            const long ib = (long)ci.b * p.M;
            if (i < p.M && j < p.N) {
              f32x4 o = v;
              if constexpr (EPI == EPI_AXPBY) {
                const f32x4 x = load4((const bf16*)p.e.aux + (i + ib) * p.e.ld_aux + j);
                o = f32x4{fmaf(p.e.alpha, x.x, p.e.beta_f * v.x), fmaf(p.e.alpha, x.y, p.e.beta_f * v.y),
                          fmaf(p.e.alpha, x.z, p.e.beta_f * v.z), fmaf(p.e.alpha, x.w, p.e.beta_f * v.w)};
                store4((bf16*)p.e.c_lp + (i + ib) * p.e.ld_lp + j, o);
              } else {
                epi_apply4<EPI>(p.e, ci.split, i + ib, j, v);
              }
              if constexpr (EPI == EPI_LP || EPI == EPI_AXPBY) {
                if (ci.mir) store_mirror(i, j, ib, o);
              }
            }
          } else {
            if (i < p.M && j < p.N && i >= ci.mlo && j >= ci.nlo)
              epi_apply4<EPI>(p.e, ci.split, i, j,
                              f32x4{acc[a][c][4 * q], acc[a][c][4 * q + 1], acc[a][c][4 * q + 2],
                                    acc[a][c][4 * q + 3]});
          }
        }
        if constexpr (EPI == EPI_F32_ACC) __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
      for (int c = 0; c < FN; ++c) acc[a][c] = f32x16{};
  };

  // ReLU² backward epilogue: the saved g of the next 32-row block is loaded
  // while the current block is computed and stored, so the load latency is
  // paid once per tile rather than once per block.
  auto epilogue_drelu2 = [&](const Item& ci) {
    u32x2 gv[2][FN][4];
    auto load_g = [&](int a, u32x2 (&dst)[FN][4]) {
      const long i = ci.m0 + wm * TM + a * 32 + (lane & 31);
#pragma unroll
      for (int c = 0; c < FN; ++c)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const long j = ci.n0 + wn * TN + c * 32 + 8 * q + 4 * (lane >> 5);
          dst[c][q] = (i < p.M && j < p.N)
                          ? *reinterpret_cast<const u32x2*>((const bf16*)p.e.aux + i * p.e.ld_aux + j)
                          : u32x2{0u, 0u};
        }
    };
    load_g(0, gv[0]);
#pragma unroll
    for (int a = 0; a < FM; ++a) {
      if (a + 1 < FM) load_g(a + 1, gv[(a + 1) & 1]);
      const long i = ci.m0 + wm * TM + a * 32 + (lane & 31);
#pragma unroll
      for (int c = 0; c < FN; ++c)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const long j = ci.n0 + wn * TN + c * 32 + 8 * q + 4 * (lane >> 5);
          const u32x2 w = gv[a & 1][c][q];
          const f32x4 g{bf16lo_to_f32(w.x), bf16hi_to_f32(w.x), bf16lo_to_f32(w.y), bf16hi_to_f32(w.y)};
          const f32x4 dg{acc[a][c][4 * q], acc[a][c][4 * q + 1], acc[a][c][4 * q + 2], acc[a][c][4 * q + 3]};
          if (i < p.M && j < p.N) store4((bf16*)p.e.c_lp + i * p.e.ld_lp + j, drelu2(dg, g));
        }
    }
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
      for (int c = 0; c < FN; ++c) acc[a][c] = f32x16{};
  };

  if constexpr (P64) {
    // One 160 KB array of five 32 KB slots.  Half i of the sequence A(0) B(0)
    // A(1) B(1) ... goes to slot i mod 5: while pair P is computed from its
    // two slots, A(P+1) is in flight or landed and the loads of B(P+1) and
    // A(P+2) fill the slots of pair P-1.  The loads are inline assembly (the
    // compiler sees none of them and adds no waits); the slot offsets change
    // every pair, so the read addresses are formed per pair from a few
    // per-lane parts and immediate offsets.
    __shared__ __attribute__((aligned(1024))) bf16 ring[5 * 16384];
    const uint32_t ring0 = (uint32_t)(uintptr_t)ring;
    auto npairs = [&](const Item& I) { return max((I.kend - I.kbeg + 63) / 64, 2); };
    auto slot_el = [](int j) { return (j >= 5 ? j - 5 : j) * 16384; };
    // per-lane parts of the fragment addresses (elements), per k-step s;
    // the 32-row block a (or c) adds a * 2048
    int la[4], lb[4];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int r = lane & 31, kc = 2 * s4 + (lane >> 5);
      la[s4] = (wm * TM + r) * 64 + ((kc ^ ((r >> 1) & 7)) << 3);
      lb[s4] = (wn * TN + r) * 64 + ((kc ^ ((r >> 1) & 7)) << 3);
    }
    auto read_pair = [&](int eA, int eB, int st, bf16x8* fa, bf16x8* fb) {
      const bf16* pa = ring + eA + la[st];
      const bf16* pb = ring + eB + lb[st];
#pragma unroll
      for (int a = 0; a < FM; ++a) fa[a] = *reinterpret_cast<const bf16x8*>(pa + a * 2048);
#pragma unroll
      for (int c = 0; c < FN; ++c) fb[c] = *reinterpret_cast<const bf16x8*>(pb + c * 2048);
    };
    // One MFMA step (16 MFMAs) interleaved with the NR fragment reads.
    auto mstep = [&](const bf16x8* fa, const bf16x8* fb) {
#pragma unroll
      for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int c = 0; c < FN; ++c)
          acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[c], fa[a], acc[a][c], 0, 0, 0);
#pragma unroll
      for (int i = 0; i < FM * FN; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      if (NR > FM * FN) __builtin_amdgcn_sched_group_barrier(0x100, NR - FM * FN, 0);
      __builtin_amdgcn_sched_barrier(0);
    };
    // scalar byte offset of this wavefront's block q = 0 of a half, and the step per q
    const uint32_t sa0 = (uint32_t)(16L * wv * p.lda), saq = (uint32_t)(64L * p.lda);
    const uint32_t sb0 = (uint32_t)(16L * wv * p.ldb), sbq = (uint32_t)(64L * p.ldb);
    // loads q0 .. q0+nq-1 of a half into the slot at element offset e
    auto load_half = [&](rsrc_t rs, uint32_t voff, uint32_t s0, uint32_t sq, int e, int q0, int nq) {
      const uint32_t m0 = ring0 + (uint32_t)e * 2u + (uint32_t)wv * 1024u;
#pragma unroll
      for (int q = q0; q < q0 + nq; ++q) dma_lds(rs, voff, s0 + (uint32_t)q * sq, m0 + (uint32_t)q * 4096u);
    };

    // bf16 epilogue staged through LDS (16 KB per wavefront at element offset
    // e): each half of the wavefront's 128 x 128 block (64 rows) is written
    // as 8-byte pieces in the accumulator layout, then read back as 16-byte
    // row chunks, so that every store covers four 256-byte row segments
    // (whole 128-byte lines) instead of 32 rows x 16 bytes.  The 16-byte
    // chunk index of row r is XOR-ed with r & 15.  A barrier at the end lets
    // the next loads into these slots go ahead.
    auto epilogue_lds = [&](const Item& I, int e) {
      bf16* st = ring + e;
      // the swizzle term, opaque to the compiler so that the sixteen staging
      // addresses are formed here rather than hoisted out of the loop (where
      // they would occupy registers for the whole kernel)
      int sw = lane & 15, sx = (lane & 15) ^ (lane >> 4);
      asm volatile("" : "+v"(sw), "+v"(sx));
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
        for (int a2 = 0; a2 < 2; ++a2) {
          const int a = 2 * hf + a2;
          const int r = a2 * 32 + (lane & 31);
#pragma unroll
          for (int c = 0; c < FN; ++c)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              f32x4 v{acc[a][c][4 * q], acc[a][c][4 * q + 1], acc[a][c][4 * q + 2], acc[a][c][4 * q + 3]};
              if constexpr (EPI == EPI_RELU2) {
                const f32x4 rl{fmaxf(v.x, 0.f), fmaxf(v.y, 0.f), fmaxf(v.z, 0.f), fmaxf(v.w, 0.f)};
                v = rl * rl;
              }
              const int ch = (4 * c + q) ^ sw;  // r & 15 == lane & 15
              *reinterpret_cast<u32x2*>(st + r * 128 + ch * 8 + 4 * (lane >> 5)) =
                  u32x2{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
            }
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          if ((t & 3) == 0) __builtin_amdgcn_sched_barrier(0);  // four reads and stores in flight
          const int r = 4 * t + (lane >> 4), ch = lane & 15;
          // r & 15 = 4 (t & 3) + lane / 16, so ch ^ (r & 15) = sx ^ 4 (t & 3)
          const u32x4 w = *reinterpret_cast<const u32x4*>(st + r * 128 + ((sx ^ (4 * (t & 3))) << 3));
          const long i = I.m0 + wm * TM + hf * 64 + r;
          const long j = I.n0 + wn * TN + ch * 8;
          bf16* dst = (bf16*)p.e.c_lp + i * p.e.ld_lp + j;
          if (i < p.M && i >= I.mlo && j >= I.nlo) {
            if (j + 8 <= p.N) {
              *reinterpret_cast<u32x4*>(dst) = w;
            } else if (j < p.N) {
              *reinterpret_cast<u32x2*>(dst) = u32x2{w.x, w.y};  // N is a multiple of 4
            }
          }
        }
      }
#pragma unroll
      for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int c = 0; c < FN; ++c) acc[a][c] = f32x16{};
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };

    // ReLU² backward staged the same way: the fp32 dg of one 32-row block
    // ([32][128] floats, 16 KB per wavefront, 16-byte chunk XOR row & 15) is
    // read back as four consecutive columns per lane, two rows per
    // instruction, and combined with g loaded in that layout (one block
    // ahead); du goes out as 8-byte pieces that cover two 256-byte row
    // segments per instruction.
    auto epilogue_drelu2_lds = [&](const Item& I, int e) {
      float* st = reinterpret_cast<float*>(ring + e);
      // opaque swizzle terms (see epilogue_lds)
      int sw = (lane & 15) ^ (lane >> 5), sy = (lane & 31) ^ (lane >> 5);
      asm volatile("" : "+v"(sw), "+v"(sy));
      const int jl = I.n0 + wn * TN + 4 * (lane & 31);
      u32x2 gv[2][16];
      auto load_g = [&](int a, u32x2 (&dst)[16]) {
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const long i = I.m0 + wm * TM + a * 32 + 2 * t + (lane >> 5);
          dst[t] = (i < p.M && jl < p.N)
                       ? *reinterpret_cast<const u32x2*>((const bf16*)p.e.aux + i * p.e.ld_aux + jl)
                       : u32x2{0u, 0u};
        }
      };
      load_g(0, gv[0]);
#pragma unroll
      for (int a = 0; a < FM; ++a) {
        if (a + 1 < FM) load_g(a + 1, gv[(a + 1) & 1]);
        // row lane & 31, chunk (8 c + 2 q + lane / 32) ^ (row & 15) = (8 c + 2 q) ^ sw
#pragma unroll
        for (int c = 0; c < FN; ++c)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *reinterpret_cast<f32x4*>(st + (lane & 31) * 128 + (((8 * c + 2 * q) ^ sw) << 2)) =
                f32x4{acc[a][c][4 * q], acc[a][c][4 * q + 1], acc[a][c][4 * q + 2], acc[a][c][4 * q + 3]};
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          if ((t & 3) == 0) __builtin_amdgcn_sched_barrier(0);
          // row 2 t + lane / 32, chunk (lane & 31) ^ (row & 15) = sy ^ (2 t & 14)
          const int r = 2 * t + (lane >> 5);
          const f32x4 dg = *reinterpret_cast<const f32x4*>(st + r * 128 + ((sy ^ ((2 * t) & 14)) << 2));
          const u32x2 w = gv[a & 1][t];
          const f32x4 g{bf16lo_to_f32(w.x), bf16hi_to_f32(w.x), bf16lo_to_f32(w.y), bf16hi_to_f32(w.y)};
          const long i = I.m0 + wm * TM + a * 32 + r;
          if (i < p.M && jl < p.N && i >= I.mlo && jl >= I.nlo)
            store4((bf16*)p.e.c_lp + i * p.e.ld_lp + jl, drelu2(dg, g));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int c = 0; c < FN; ++c) acc[a][c] = f32x16{};
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };

    int it = wfirst;
    Item ci = item(it);
    int nit = it + G;
    bool has_next = nit < nitems;
    Item nx = item(has_next ? nit : it);
    uint32_t va = pair_voff(p.lda, ci.m0, wv, lane), vb = pair_voff(p.ldb, ci.n0, wv, lane);
    uint32_t na = pair_voff(p.lda, nx.m0, wv, lane), nb = pair_voff(p.ldb, nx.n0, wv, lane);
    // half of pair PP of the current item (PP < np) or of the next one (PP - np)
    auto rs_half = [&](bool isA, int np, int PP) {
      const bool cur = PP < np;
      const int q = cur ? PP : PP - np;
      const int kbeg = cur ? ci.kbeg : nx.kbeg, klen = cur ? ci.kend - ci.kbeg : nx.kend - nx.kbeg;
      const bool live = (cur || has_next) && q < (klen + 63) / 64;
      return isA ? slice_rsrc(p.A, p.a_bytes, a_kstep, kbeg + 64 * q, live)
                 : slice_rsrc(p.B, p.b_bytes, b_kstep, kbeg + 64 * q, live);
    };
    int np = npairs(ci);
    // prologue: A(0), B(0), A(1); wait for the first two
    load_half(rs_half(true, np, 0), va, sa0, saq, 0, 0, 8);
    load_half(rs_half(false, np, 0), vb, sb0, sbq, 16384, 0, 8);
    load_half(rs_half(true, np, 1), va, sa0, saq, 32768, 0, 8);
    asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
    read_pair(0, 16384, 0, fa0, fb0);
    int cs = 0;  // slot of A(P); B(P) is in cs+1, A(P+1) in cs+2 (mod 5)
    for (;;) {
      for (int P = 0; P < np; ++P) {
        const int eA = slot_el(cs), eB = slot_el(cs + 1), eA1 = slot_el(cs + 2), eB1 = slot_el(cs + 3),
                  eDA = slot_el(cs + 4);
        const rsrc_t rb1 = rs_half(false, np, P + 1), ra2 = rs_half(true, np, P + 2);
        const uint32_t vb1 = P + 1 < np ? vb : nb, va2 = P + 2 < np ? va : na;
        // B(P+1) with the first step, A(P+2) with the next two; before the
        // last step wait for everything but A(P+2) (8 loads): the barrier
        // publishes pair P+1 and frees the slots of pair P
        bf16x8 fa1[FM], fb1[FN];
        load_half(rb1, vb1, sb0, sbq, eB1, 0, 8);
        read_pair(eA, eB, 1, fa1, fb1);
        mstep(fa0, fb0);
        load_half(ra2, va2, sa0, saq, eDA, 0, 4);
        read_pair(eA, eB, 2, fa0, fb0);
        mstep(fa1, fb1);
        load_half(ra2, va2, sa0, saq, eDA, 4, 4);
        read_pair(eA, eB, 3, fa1, fb1);
        mstep(fa0, fb0);
        asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        read_pair(eA1, eB1, 0, fa0, fb0);
        mstep(fa1, fb1);
        cs = cs >= 3 ? cs - 3 : cs + 2;
      }
      if constexpr (EPI == EPI_LP || EPI == EPI_RELU2) {
        // the two slots of the pair just finished are free until the next
        // item's first pair loads into them
        epilogue_lds(ci, slot_el(wv < 2 ? cs + 3 : cs + 4) + (wv & 1) * 8192);
      } else if constexpr (EPI == EPI_DRELU2) {
        epilogue_drelu2_lds(ci, slot_el(wv < 2 ? cs + 3 : cs + 4) + (wv & 1) * 8192);
      } else {
        epilogue(ci);
      }
      if (!has_next) break;
      it = nit;
      ci = nx;
      va = na;
      vb = nb;
      np = npairs(ci);
      nit = it + G;
      has_next = nit < nitems;
      nx = item(has_next ? nit : it);
      na = pair_voff(p.lda, nx.m0, wv, lane);
      nb = pair_voff(p.ldb, nx.n0, wv, lane);
    }
    wait_vmem();  // the final no-op loads still target LDS
    return;
  } else {
  // four LDS stages per operand, as separate objects so that the compiler can
  // tell the in-flight LDS-direct loads (into three stages) from the fragment
  // reads (of the fourth) and does not wait on them
  __shared__ __attribute__((aligned(1024))) bf16 As0[BM * kBK];
  __shared__ __attribute__((aligned(1024))) bf16 As1[BM * kBK];
  __shared__ __attribute__((aligned(1024))) bf16 As2[BM * kBK];
  __shared__ __attribute__((aligned(1024))) bf16 As3[BM * kBK];
  __shared__ __attribute__((aligned(1024))) bf16 Bs0[BN * kBK];
  __shared__ __attribute__((aligned(1024))) bf16 Bs1[BN * kBK];
  __shared__ __attribute__((aligned(1024))) bf16 Bs2[BN * kBK];
  __shared__ __attribute__((aligned(1024))) bf16 Bs3[BN * kBK];

  int it = wfirst;
  Item ci = item(it);
  uint32_t va[4], vb[4];
  item_voff(ci, va, vb);
  // prologue: the first three slices, then the first fragments
  load_slice(As0, Bs0, va, vb, ci, 0);
  load_slice(As1, Bs1, va, vb, ci, 1);
  load_slice(As2, Bs2, va, vb, ci, 2);
  wait_first_slice_and_sync();
  read_step(As0, Bs0, 0, fa0, fb0);

  // Slice in stage S; the next slice is in stage S+1 and the loads go to S+3 (mod 4).
#define NC_STEP(S, S1, S3, VA, VB, IT, J, ALIVE) \
  compute(As##S, Bs##S, As##S1, Bs##S1, As##S3, Bs##S3, VA, VB, IT, J, ALIVE);

  // Work items in turn.  Each runs a multiple of four 32-deep slices (stage i
  // holds slices i, i+4, ...); missing slices load zeros and add exactly 0.
  // The last slices of an item prefetch the first three of the next item, so
  // only the very first slices wait for their loads.
  for (;;) {
    const int nk4 = (max(ci.nk, 1) + 3) & ~3;
    const int nit = it + G;
    const bool has_next = nit < nitems;
    const Item nx = has_next ? item(nit) : ci;
    int kt = 0;
    for (; kt + 4 < nk4; kt += 4) {
      NC_STEP(0, 1, 3, va, vb, ci, kt + 3, true)
      NC_STEP(1, 2, 0, va, vb, ci, kt + 4, true)
      NC_STEP(2, 3, 1, va, vb, ci, kt + 5, true)
      NC_STEP(3, 0, 2, va, vb, ci, kt + 6, true)
    }
    // last four slices: after the item's own slice kt + 3, prefetch the next item
    NC_STEP(0, 1, 3, va, vb, ci, kt + 3, true)
    uint32_t na[4], nb[4];
    item_voff(nx, na, nb);
    NC_STEP(1, 2, 0, na, nb, nx, 0, has_next)
    NC_STEP(2, 3, 1, na, nb, nx, 1, has_next)
    NC_STEP(3, 0, 2, na, nb, nx, 2, has_next)
    if constexpr (EPI == EPI_DRELU2) epilogue_drelu2(ci);
    else epilogue(ci);
    if (!has_next) break;
    it = nit;
    ci = nx;
    va[0] = na[0]; va[1] = na[1]; va[2] = na[2]; va[3] = na[3];
    vb[0] = nb[0]; vb[1] = nb[1]; vb[2] = nb[2]; vb[3] = nb[3];
  }
#undef NC_STEP
  wait_vmem();  // the final no-op loads still target LDS
  }
}

// ------------------------------------------------------------------ SIMT fp32 path
template <bool KMAJ>
__device__ __forceinline__ float ld_op(const float* g, long ld, int row, int k, int rows_lim, int k_lim) {
  if (row >= rows_lim || k >= k_lim) return 0.f;
  return KMAJ ? g[(size_t)row * ld + k] : g[(size_t)k * ld + row];
}

template <bool AK, bool BKM, int EPI>
__global__ void __launch_bounds__(256) gemm_simt_kernel(GemmParams p) {
  __shared__ float As[16][65];
  __shared__ float Bs[16][65];
  const int tm = blockIdx.x / p.tiles_n, tn = blockIdx.x % p.tiles_n;
  const int m0 = tm * 64, n0 = tn * 64;
  const int split = blockIdx.z;
  const int bb = blockIdx.y;  // batch member
  const int kbeg = split * p.kchunk;
  const int kend = min(p.K, kbeg + p.kchunk);
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {};
  const float* Ag = (const float*)((const char*)p.A + bb * p.a_bs);
  const float* Bg = (const float*)((const char*)p.B + bb * p.b_bs);
  for (int k0 = kbeg; k0 < kend; k0 += 16) {
    for (int e = threadIdx.x; e < 64 * 16; e += 256) {
      int r, kk;
      if (AK) { r = e >> 4; kk = e & 15; } else { kk = e >> 6; r = e & 63; }
      As[kk][r] = ld_op<AK>(Ag, p.lda, m0 + r, k0 + kk, p.M, kend);
      if (BKM) { r = e >> 4; kk = e & 15; } else { kk = e >> 6; r = e & 63; }
      Bs[kk][r] = ld_op<BKM>(Bg, p.ldb, n0 + r, k0 + kk, p.N, kend);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) { a[q] = As[kk][ty * 4 + q]; b[q] = Bs[kk][tx * 4 + q]; }
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = fmaf(a[x], b[y], acc[x][y]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const long i = m0 + ty * 4 + x, j = n0 + tx * 4 + y;
      if (i < p.M && j < p.N) epi_apply<EPI, float>(p.e, split, i + (long)bb * p.M, j, acc[x][y]);
    }
}

// ------------------------------------------------------------------ transpose
// 64 x 64 tiles through LDS.  Full tiles with 16-byte aligned rows move
// 16-byte pieces (a thread loads two 8-element row chunks and stores two
// 8-element chunks of a transposed row); edge tiles move single elements.
__global__ void __launch_bounds__(256) transpose_bf16_kernel(const bf16* __restrict__ src, int R, int C, long lds,
                                                             bf16* __restrict__ dst, long ldd, int vec) {
  __shared__ __attribute__((aligned(16))) bf16 tile[64][72];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int t = threadIdx.x;
  if (vec && r0 + 64 <= R && c0 + 64 <= C) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int r = t / 8 + 32 * k, ch = t % 8;
      *reinterpret_cast<u32x4*>(&tile[r][ch * 8]) =
          *reinterpret_cast<const u32x4*>(src + (size_t)(r0 + r) * lds + c0 + ch * 8);
    }
    __syncthreads();
    const int c = t / 4, rb = (t % 4) * 16;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      bf16x8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = tile[rb + 8 * k + e][c];
      *reinterpret_cast<u32x4*>(dst + (size_t)(c0 + c) * ldd + r0 + rb + 8 * k) = __builtin_bit_cast(u32x4, v);
    }
    return;
  }
  const int tx = t & 63, ty = t >> 6;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int r = r0 + ty * 16 + k, c = c0 + tx;
    if (r < R && c < C) tile[ty * 16 + k][tx] = src[(size_t)r * lds + c];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int c = c0 + ty * 16 + k, r = r0 + tx;
    if (r < R && c < C) dst[(size_t)c * ldd + r] = tile[tx][ty * 16 + k];
  }
}

int launch_transpose_bf16(const void* src, int R, int C, long lds, void* dst, long ldd, hipStream_t s) {
  if (R <= 0 || C <= 0) return 0;
  dim3 grid((unsigned)((C + 63) / 64), (unsigned)((R + 63) / 64));
  const int vec = ((uintptr_t)src % 16 == 0 && (uintptr_t)dst % 16 == 0 && lds % 8 == 0 && ldd % 8 == 0) ? 1 : 0;
  transpose_bf16_kernel<<<grid, 256, 0, s>>>((const bf16*)src, R, C, lds, (bf16*)dst, ldd, vec);
  NC_LAUNCH_CHECK();
  return 0;
}

// ------------------------------------------------------------------ split-K reduce
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float* __restrict__ part, int splits, long MN,
                                                            int M, int N, float* __restrict__ out, long ldc,
                                                            int beta) {
  const long idx4 = ((long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (idx4 >= MN) return;
  const long i = idx4 / N, j = idx4 - i * N;
  f32x4 s = *reinterpret_cast<const f32x4*>(part + idx4);
  for (int q = 1; q < splits; ++q) s += *reinterpret_cast<const f32x4*>(part + (size_t)q * MN + idx4);
  f32x4* o = reinterpret_cast<f32x4*>(out + i * ldc + j);
  if (beta) s += *o;
  *o = s;
}

// ------------------------------------------------------------------ host dispatch
template <int EPI, bool KTAIL, bool BAT>
static void launch_mfma_k(const GemmParams& p, bool ak, bool bk, bool p64, dim3 grid, hipStream_t s) {
  if constexpr (!KTAIL && !BAT) {
    if (p64 && ak && bk) {
      gemm_mfma_kernel<true, true, EPI, false, false, true><<<grid, 256, 0, s>>>(p);
      return;
    }
  }
  if (ak && bk) gemm_mfma_kernel<true, true, EPI, KTAIL, BAT, false><<<grid, 256, 0, s>>>(p);
  else if (ak) gemm_mfma_kernel<true, false, EPI, KTAIL, BAT, false><<<grid, 256, 0, s>>>(p);
  else if (bk) gemm_mfma_kernel<false, true, EPI, KTAIL, BAT, false><<<grid, 256, 0, s>>>(p);
  else gemm_mfma_kernel<false, false, EPI, KTAIL, BAT, false><<<grid, 256, 0, s>>>(p);
}
// The 64-deep pair loop serves products whose operands are both
// k-contiguous (the forward products and the LM-head logits; measured 5-10%
// faster there, no gain or a loss where B is m-contiguous, whose rows are
// already 512 bytes) with K a multiple of 64 of at least 640 and row
// strides of at least K.  Its last tile-row and tile-column are moved back
// inside the operands, so M and N are at least 256; N is a multiple of 8
// (whole 16-byte column chunks in the staged epilogues).
static bool use_pairs(const GemmParams& p, bool ak, bool bk) {
  return ak && bk && p.batch == 1 && !p.sym && p.K % 64 == 0 && p.K >= 640 && p.lda >= p.K && p.ldb >= p.K &&
         p.M >= 256 && p.N >= 256 && p.N % 8 == 0;
}
template <int EPI, bool KTAIL>
static int launch_mfma_b(const GemmParams& p, bool ak, bool bk, dim3 grid, hipStream_t s) {
  if (p.batch == 1 && !p.sym) {
    launch_mfma_k<EPI, KTAIL, false>(p, ak, bk, !KTAIL && use_pairs(p, ak, bk), grid, s);
    return 0;
  }
  if constexpr (EPI == EPI_LP || EPI == EPI_AXPBY || EPI == EPI_F32) {
    launch_mfma_k<EPI, KTAIL, true>(p, ak, bk, false, grid, s);
    return 0;
  }
  return NC_ERR_UNSUPPORTED;
}
// A k-contiguous operand with K % 32 != 0 needs the per-lane cut of the last
// slice; the model's layers never do (their widths are multiples of 64), so
// only the fp32-output products (the general matrix-product entry point) and
// the Newton-Schulz combination (EPI_AXPBY) carry that variant.
template <int EPI>
static int launch_mfma(const GemmParams& p, bool ak, bool bk, dim3 grid, hipStream_t s) {
  const bool ktail = (ak || bk) && (p.K % kBK) != 0;
  if (!ktail) return launch_mfma_b<EPI, false>(p, ak, bk, grid, s);
  if constexpr (EPI == EPI_F32 || EPI == EPI_F32_ACC || EPI == EPI_AXPBY) return launch_mfma_b<EPI, true>(p, ak, bk, grid, s);
  return NC_ERR_UNSUPPORTED;
}

template <int EPI>
static void launch_simt(const GemmParams& p, bool ak, bool bk, dim3 grid, hipStream_t s) {
  if (ak && bk) gemm_simt_kernel<true, true, EPI><<<grid, 256, 0, s>>>(p);
  else if (ak) gemm_simt_kernel<true, false, EPI><<<grid, 256, 0, s>>>(p);
  else if (bk) gemm_simt_kernel<false, true, EPI><<<grid, 256, 0, s>>>(p);
  else gemm_simt_kernel<false, false, EPI><<<grid, 256, 0, s>>>(p);
}

// Compute units of the current device (cached per device).
static int num_cus() {
  static int cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cache[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// K splits of the fp32-output product (1 = none).  bf16 path (persistent,
// one workgroup per compute unit): the split count minimizing the serial
// work of the busiest workgroup, rounds x K-chunk, plus the time of writing
// and reducing the fp32 partials (in the same units: one unit is one k of
// a 256 x 256 tile, ~ M N / 21000 units per split); ties go to fewer splits.
int gemm_splits(int M, int N, int K, int dtype) {
  if (K < 2048) return 1;
  if (dtype != 0) {
    const long tiles = (long)((M + 63) / 64) * ((N + 63) / 64);
    if (tiles >= 512) return 1;
    int s = (int)((1024 + tiles - 1) / tiles);
    s = std::min(s, std::min(K / 1024, 32));
    return s < 1 ? 1 : s;
  }
  const long tiles = (long)((M + 255) / 256) * ((N + 255) / 256);
  const long cus = num_cus();
  const int smax = std::min(32, K / 1024);
  int best = 1;
  double best_cost = 0;
  for (int s = 1; s <= smax; ++s) {
    const long kc = ((K + s - 1) / s + 127) / 128 * 128;
    const long ss = (K + kc - 1) / kc;
    const long rounds = (tiles * ss + cus - 1) / cus;
    const double cost = (double)rounds * kc + (ss > 1 ? (double)ss * M * N / 21000.0 : 0.0);
    if (s == 1 || cost < best_cost) {
      best = s;
      best_cost = cost;
    }
  }
  return best;
}

uint64_t gemm_ws_bytes(int M, int N, int K, int dtype) {
  const int s = gemm_splits(M, N, K, dtype);
  return s > 1 ? (uint64_t)s * M * N * 4 : 0;
}

// Tile-rows per group of the persistent tile walk (items go down a group of
// tile-rows, then across the columns, so that one XCD's workgroups share A
// rows and B columns in its L2).  Swept over 1..32 on every product of the
// depth-20 step: very wide outputs (the LM-head logits, 256 column tiles)
// run 1.7x faster walking one tile-row at a time; elsewhere 4 is within 2%
// of the best (and 1.2x better than 8 on the Wo weight gradient).
static int gemm_group(int tiles_m, int tiles_n, int splits) {
  (void)tiles_m;
  (void)splits;
  return tiles_n >= 64 ? 1 : 4;
}

int launch_gemm(const GemmCall& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return 0;
  const int t = g.dtype == 0 ? 256 : 64;
  GemmParams p;
  p.A = g.A; p.B = g.B; p.lda = g.lda; p.ldb = g.ldb;
  {
    // operand extents in bytes; the buffer loads need them below 2^31
    const uint64_t es = g.dtype == 0 ? 2 : 4;
    const uint64_t ra = g.a_k ? (uint64_t)g.M : (uint64_t)g.K, ca = g.a_k ? (uint64_t)g.K : (uint64_t)g.M;
    const uint64_t rb = g.b_k ? (uint64_t)g.N : (uint64_t)g.K, cb = g.b_k ? (uint64_t)g.K : (uint64_t)g.N;
    const uint64_t ab = ra ? ((ra - 1) * g.lda + ca) * es : 0, bb = rb ? ((rb - 1) * g.ldb + cb) * es : 0;
    if (ab >= kOOB || bb >= kOOB) return NC_ERR_UNSUPPORTED;
    p.a_bytes = (uint32_t)ab;
    p.b_bytes = (uint32_t)bb;
  }
  p.M = g.M; p.N = g.N; p.K = g.K;
  p.tiles_m = (g.M + t - 1) / t;
  p.tiles_n = (g.N + t - 1) / t;
  p.e = g.e;
  if (g.batch < 1) return NC_ERR_ARG;
  const bool batched = g.batch > 1;
  if (batched && !(g.epi == EPI_LP || g.epi == EPI_AXPBY || (g.epi == EPI_F32 && !g.e.beta)))
    return NC_ERR_UNSUPPORTED;
  p.batch = g.batch;
  // symmetric results: MFMA path only (the fp32 path computes every tile)
  if (g.sym && (g.M != g.N || !(g.epi == EPI_LP || g.epi == EPI_AXPBY))) return NC_ERR_UNSUPPORTED;
  p.sym = g.sym && g.dtype == 0;
  p.a_bs = g.a_bstride * (g.dtype == 0 ? 2 : 4);
  p.b_bs = g.b_bstride * (g.dtype == 0 ? 2 : 4);
  int splits = 1;
  if (g.epi == EPI_F32 && g.splitk_ws && !batched) splits = gemm_splits(g.M, g.N, g.K, g.dtype);
  int kchunk = g.K;
  if (splits > 1) {
    // chunks of a multiple of four 32-deep slices (the kernel runs them in fours)
    kchunk = ((g.K + splits - 1) / splits + 4 * kBK - 1) / (4 * kBK) * (4 * kBK);
    splits = (g.K + kchunk - 1) / kchunk;
    if ((uint64_t)splits * g.M * g.N * 4 > g.splitk_bytes) {
      splits = 1;
      kchunk = g.K;
    }
  }
  if (splits > 1) {
    p.e.c32 = g.splitk_ws;
    p.e.ldc = g.N;
    p.e.beta = 0;
    p.e.split_stride = (long)g.M * g.N;
  }
  p.kchunk = kchunk > 0 ? kchunk : 1;
  p.splits = splits;
  p.group = gemm_group(p.tiles_m, p.tiles_n, splits);
  dim3 grid(p.tiles_m * p.tiles_n, g.batch, splits);
  if (g.dtype == 0) {
    // persistent: one workgroup per compute unit (each holds 128 KB of LDS)
    const long tiles = p.sym ? (long)p.tiles_m * (p.tiles_m + 1) / 2 : (long)p.tiles_m * p.tiles_n;
    const long items = tiles * splits * g.batch;
    grid = dim3((unsigned)std::min<long>(items, num_cus()), 1, 1);
  }
  // K == 0 runs the kernels with an empty k-loop: the epilogue sees zeros.
  if (g.dtype == 0) {
    int rc = 0;
    switch (g.epi) {
      case EPI_F32:
        // accumulation into C gets its own kernel (the C loads need registers)
        rc = p.e.beta ? launch_mfma<EPI_F32_ACC>(p, g.a_k, g.b_k, grid, s) : launch_mfma<EPI_F32>(p, g.a_k, g.b_k, grid, s);
        break;
      case EPI_RESID: rc = launch_mfma<EPI_RESID>(p, g.a_k, g.b_k, grid, s); break;
      case EPI_LP: rc = launch_mfma<EPI_LP>(p, g.a_k, g.b_k, grid, s); break;
      case EPI_RELU2: rc = launch_mfma<EPI_RELU2>(p, g.a_k, g.b_k, grid, s); break;
      case EPI_DRELU2: rc = launch_mfma<EPI_DRELU2>(p, g.a_k, g.b_k, grid, s); break;
      case EPI_AXPBY: rc = launch_mfma<EPI_AXPBY>(p, g.a_k, g.b_k, grid, s); break;
      default: return 8;
    }
    if (rc) return rc;
  } else {
    switch (g.epi) {
      case EPI_F32: launch_simt<EPI_F32>(p, g.a_k, g.b_k, grid, s); break;
      case EPI_RESID: launch_simt<EPI_RESID>(p, g.a_k, g.b_k, grid, s); break;
      case EPI_LP: launch_simt<EPI_LP>(p, g.a_k, g.b_k, grid, s); break;
      case EPI_RELU2: launch_simt<EPI_RELU2>(p, g.a_k, g.b_k, grid, s); break;
      case EPI_DRELU2: launch_simt<EPI_DRELU2>(p, g.a_k, g.b_k, grid, s); break;
      case EPI_AXPBY: launch_simt<EPI_AXPBY>(p, g.a_k, g.b_k, grid, s); break;
      default: return 8;
    }
  }
  NC_LAUNCH_CHECK();
  if (splits > 1) {
    const long MN = (long)g.M * g.N;
    splitk_reduce_kernel<<<(unsigned)((MN / 4 + 255) / 256), 256, 0, s>>>(g.splitk_ws, splits, MN, g.M, g.N,
                                                                          g.e.c32, g.e.ldc, g.e.beta);
    NC_LAUNCH_CHECK();
  }
  return 0;
}

}  // namespace nc
