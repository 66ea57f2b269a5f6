// Matrix products for every linear layer of the model:
//   C[i, j] = sum_k A(i, k) * B(j, k)
// forward y = x W^T (both operands k-contiguous), input gradient dx = dy W
// (B is W stored [k][j]) and weight gradient dW = dy^T x (both operands
// stored [k][i]); see "nanochat explainer", Modern architecture choices, for
// the layers (QKV and output projections, ReLU² MLP, untied LM head).
//
// bf16 path: v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  A 256-thread
// workgroup owns a 256x256 output tile; its four wavefronts each own 128x128
// (4x4 MFMA blocks of 32x32).  K advances 64 at a time through two LDS
// buffers (the next tile's global loads are in flight while the current one
// is multiplied).  LDS rows are 64 bf16 (128 B) with the 16-byte chunk index
// XOR-swizzled by (row & 7), so the MFMA fragment reads (one 16-byte chunk per
// lane, 32 consecutive rows) are bank-conflict free.  Operands whose
// reduction index is not contiguous in memory are loaded as 8x8 bf16 blocks
// and transposed in registers before the LDS store.
//
// fp32 debug path: a plain 64x64 LDS-tiled SIMT kernel with the same epilogues.
//
// Epilogues are fused so that each output is written once: fp32 store or
// accumulate, bf16 store, residual add into the fp32 stream, ReLU² (stores
// u and g = max(u,0)^2), and the ReLU² backward (du = dg * 2 max(u,0)).
#include "common.h"
#include "kernels.h"

namespace nc {

struct GemmParams {
  const void* A;
  const void* B;
  long lda, ldb;
  uint32_t a_bytes, b_bytes;  // extent of each operand (buffer bound; beyond it loads read 0)
  int M, N, K;
  int kchunk;  // K range per split (multiple of 64)
  int tiles_m, tiles_n;
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

template <int EPI, class T>
__device__ __forceinline__ void epi_apply4(const EpiArgs& e, int split, long i, long j, f32x4 v) {
  if constexpr (EPI == EPI_F32) {
    f32x4* c = reinterpret_cast<f32x4*>(e.c32 + (size_t)split * e.split_stride + i * e.ldc + j);
    if (e.beta) v += *c;
    *c = v;
  } else if constexpr (EPI == EPI_RESID) {
    f32x4* c = reinterpret_cast<f32x4*>(e.c32 + i * e.ldc + j);
    *c = *c + v;
  } else if constexpr (EPI == EPI_LP) {
    store4((T*)e.c_lp + i * e.ld_lp + j, v);
  } else if constexpr (EPI == EPI_RELU2) {
    store4((T*)e.c_lp + i * e.ld_lp + j, v);
    const f32x4 r{fmaxf(v.x, 0.f), fmaxf(v.y, 0.f), fmaxf(v.z, 0.f), fmaxf(v.w, 0.f)};
    store4((T*)e.c_lp2 + i * e.ld_lp + j, r * r);
  } else if constexpr (EPI == EPI_DRELU2) {
    const f32x4 u = load4((const T*)e.aux + i * e.ld_aux + j);
    const f32x4 du{u.x > 0.f ? 2.f * u.x * v.x : 0.f, u.y > 0.f ? 2.f * u.y * v.y : 0.f,
                   u.z > 0.f ? 2.f * u.z * v.z : 0.f, u.w > 0.f ? 2.f * u.w * v.w : 0.f};
    store4((T*)e.c_lp + i * e.ld_lp + j, du);
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
    ((T*)e.c_lp)[i * e.ld_lp + j] = from_f32<T>(v);
    const float r = v > 0.f ? v : 0.f;
    ((T*)e.c_lp2)[i * e.ld_lp + j] = from_f32<T>(r * r);
  } else if constexpr (EPI == EPI_DRELU2) {
    const float u = to_f32(((const T*)e.aux)[i * e.ld_aux + j]);
    ((T*)e.c_lp)[i * e.ld_lp + j] = from_f32<T>(u > 0.f ? 2.f * u * v : 0.f);
  }
}

// ------------------------------------------------------------------ MFMA path
constexpr int kBK = 64;
constexpr uint32_t kOOB = 0x80000000u;  // buffer offset past every operand: loads return 0

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef short v4i16 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// LDS element offset of the 16-byte chunk `kc` (0..7) of row `row` in a
// k-contiguous [256][64] tile.  The chunk index is XOR-ed with
// (row ^ row >> 3) & 7: any 8 consecutive rows get 8 different chunk slots of
// a 128-byte bank window, and the even (and the odd) rows of any 16
// consecutive rows get 8 different slots, so a 16-byte-per-lane fragment read
// is conflict free whether the LDS serves 8 or 16 lanes per cycle.
__device__ __forceinline__ int swf(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int swz(int row, int kc) { return row * 64 + ((kc ^ swf(row)) << 3); }

// m-contiguous tiles XOR the 16-byte chunk index with this function of (k & 3):
// the four k-rows of a transposed read then land in four different 64-byte
// quarters of a 256-byte bank window (bits 2-3) and, pairwise, in different
// halves of a 128-byte window (bits 1-2), so the reads are conflict free
// whether 16 or 32 lanes are served per cycle.
__device__ __forceinline__ int swk(int k) { const int r = k & 3; return 4 * r + 2 * ((r >> 1) & 1); }

// Stage 1 KB (one wavefront instruction, 64 x 16 B) of a 64-deep K slice of a
// 256-row operand into LDS with an LDS-direct buffer load.  The LDS slots of
// one instruction are consecutive, so every lane picks the global chunk that
// belongs at its slot.  k-contiguous operands land as [256 rows][64 k] (chunk
// swizzle swf); m-contiguous operands land as [64 k][256 m] (chunk swizzle
// swk).  `b` (0..31, wave-uniform) selects the 1 KB block; `live` = false
// turns the load into a no-op read of zeros.
template <bool KMAJ>
__device__ __forceinline__ void dma_block(rsrc_t rs, long ld, int row0, int k0, int rows_lim, int k_lim,
                                          bf16* lds, int b, int lane, bool live) {
  uint32_t off;
  if constexpr (KMAJ) {
    const int row = b * 8 + (lane >> 3);
    const int kc = (lane & 7) ^ swf(row);
    const int gr = row0 + row, gk = k0 + kc * 8;
    off = (live && gr < rows_lim && gk < k_lim) ? (uint32_t)(((long)gr * ld + gk) * 2) : kOOB;
  } else {
    const int k = 2 * b + (lane >> 5);
    const int mc = (lane & 31) ^ swk(k);
    const int gk = k0 + k, gm = row0 + mc * 8;
    off = (live && gk < k_lim && gm < rows_lim) ? (uint32_t)(((long)gk * ld + gm) * 2) : kOOB;
  }
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(lds + b * 512), 16, off, 0, 0, 0);
}

__device__ __forceinline__ v4i16 tr16(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)p);
}

// MFMA 32x32x16 operand fragment for tile rows rb..rb+31 and k-step s:
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

template <bool AK, bool BKM, int EPI>
__global__ void __launch_bounds__(256, 1) gemm_mfma_kernel(GemmParams p) {
  constexpr int BM = 256, BN = 256, WM = 2, WN = 2;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  // two LDS stages per operand, as four separate objects so that the
  // compiler can tell the in-flight LDS-direct loads (into one stage) from the
  // fragment reads (of the other) and does not wait on the loads
  __shared__ __attribute__((aligned(1024))) bf16 As0[BM * kBK];
  __shared__ __attribute__((aligned(1024))) bf16 As1[BM * kBK];
  __shared__ __attribute__((aligned(1024))) bf16 Bs0[BN * kBK];
  __shared__ __attribute__((aligned(1024))) bf16 Bs1[BN * kBK];

  // Tile order: workgroup ids are dealt round-robin to the 8 XCDs; give each
  // XCD a contiguous run of logical tiles, walked in column groups of 8
  // tile-rows so that neighbours share A rows and B rows in the XCD's L2.
  const int ntiles = p.tiles_m * p.tiles_n;
  int b = blockIdx.x;
  if ((ntiles & 7) == 0) b = (b & 7) * (ntiles >> 3) + (b >> 3);
  constexpr int GROUP = 8;
  const int group_span = GROUP * p.tiles_n;
  const int grp = b / group_span;
  const int first_m = grp * GROUP;
  const int gsize = min(p.tiles_m - first_m, GROUP);
  const int tm = first_m + (b % group_span) % gsize;
  const int tn = (b % group_span) / gsize;

  const int m0 = tm * BM, n0 = tn * BN;
  const int split = blockIdx.z;
  const int kbeg = split * p.kchunk;
  const int kend = min(p.K, kbeg + p.kchunk);
  const int nk = (kend - kbeg + kBK - 1) / kBK;

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wv / WN, wn = wv % WN;
  const rsrc_t ra = make_rsrc(p.A, p.a_bytes);
  const rsrc_t rb = make_rsrc(p.B, p.b_bytes);

  f32x16 acc[FM][FN];
#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int c = 0; c < FN; ++c) acc[a][c] = f32x16{};

  // One staged 64-deep K slice: four 16-deep MFMA steps.  While step s
  // multiplies, the fragments of step s + 1 are read from LDS and a quarter of
  // the next slice's LDS-direct loads (2 blocks of A, 2 of B per wave) are
  // issued into the other buffer; sched_group_barrier interleaves the three
  // instruction streams so that the matrix cores are never left waiting for
  // their issue.
  auto compute = [&](const bf16* as, const bf16* bs, bf16* an, bf16* bn, int k_next, bool live) {
    bf16x8 af[2][FM], bfr[2][FN];
#pragma unroll
    for (int a = 0; a < FM; ++a) af[0][a] = read_frag<AK>(as, wm * TM + a * 32, 0, lane);
#pragma unroll
    for (int c = 0; c < FN; ++c) bfr[0][c] = read_frag<BKM>(bs, wn * TN + c * 32, 0, lane);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      const int cur = s & 1;
      if (s + 1 < kBK / 16) {
#pragma unroll
        for (int a = 0; a < FM; ++a) af[cur ^ 1][a] = read_frag<AK>(as, wm * TM + a * 32, s + 1, lane);
#pragma unroll
        for (int c = 0; c < FN; ++c) bfr[cur ^ 1][c] = read_frag<BKM>(bs, wn * TN + c * 32, s + 1, lane);
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        dma_block<AK>(ra, p.lda, m0, k_next, p.M, kend, an, wv * 8 + 2 * s + q, lane, live);
        dma_block<BKM>(rb, p.ldb, n0, k_next, p.N, kend, bn, wv * 8 + 2 * s + q, lane, live);
      }
#pragma unroll
      for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int c = 0; c < FN; ++c)
          acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[cur][c], af[cur][a], acc[a][c], 0, 0, 0);
      // interleave: MFMA, LDS read, MFMA, LDS read, ... with the 4 LDS-direct loads spread out
      // LDS read instructions per step (none are left on the last step; its
      // read groups stay empty)
      constexpr int NR = (AK ? FM : 2 * FM) + (BKM ? FN : 2 * FN);
#pragma unroll
      for (int i = 0; i < FM * FN; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if ((i & 3) == 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      if (NR > FM * FN) __builtin_amdgcn_sched_group_barrier(0x100, NR - FM * FN, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (nk > 0) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      dma_block<AK>(ra, p.lda, m0, kbeg, p.M, kend, As0, wv * 8 + q, lane, true);
      dma_block<BKM>(rb, p.ldb, n0, kbeg, p.N, kend, Bs0, wv * 8 + q, lane, true);
    }
  }
  wait_vmem();
  __syncthreads();
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    compute(As0, Bs0, As1, Bs1, kbeg + (kt + 1) * kBK, true);
    wait_vmem();
    __syncthreads();
    compute(As1, Bs1, As0, Bs0, kbeg + (kt + 2) * kBK, kt + 2 < nk);
    wait_vmem();
    __syncthreads();
  }
  if (kt < nk) {
    compute(As0, Bs0, As1, Bs1, kbeg + (kt + 1) * kBK, false);
    wait_vmem();  // the tail's no-op loads still target LDS
  }

  // Epilogue.  The MFMA computed C^T blocks (B fragment as the row operand), so
  // a lane holds output row m = lane & 31 of its block and, in register
  // group q = r / 4, the four consecutive columns 8 q + 4 (lane / 32) + 0..3.
#pragma unroll
  for (int a = 0; a < FM; ++a) {
    const long i = m0 + wm * TM + a * 32 + (lane & 31);
    if (i >= p.M) continue;
#pragma unroll
    for (int c = 0; c < FN; ++c)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const long j = n0 + wn * TN + c * 32 + 8 * q + 4 * (lane >> 5);
        if (j < p.N)
          epi_apply4<EPI, bf16>(p.e, split, i, j,
                                f32x4{acc[a][c][4 * q], acc[a][c][4 * q + 1], acc[a][c][4 * q + 2], acc[a][c][4 * q + 3]});
      }
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
  const int kbeg = split * p.kchunk;
  const int kend = min(p.K, kbeg + p.kchunk);
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {};
  const float* Ag = (const float*)p.A;
  const float* Bg = (const float*)p.B;
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
      if (i < p.M && j < p.N) epi_apply<EPI, float>(p.e, split, i, j, acc[x][y]);
    }
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
template <int EPI>
static void launch_mfma(const GemmParams& p, bool ak, bool bk, dim3 grid, hipStream_t s) {
  if (ak && bk) gemm_mfma_kernel<true, true, EPI><<<grid, 256, 0, s>>>(p);
  else if (ak) gemm_mfma_kernel<true, false, EPI><<<grid, 256, 0, s>>>(p);
  else if (bk) gemm_mfma_kernel<false, true, EPI><<<grid, 256, 0, s>>>(p);
  else gemm_mfma_kernel<false, false, EPI><<<grid, 256, 0, s>>>(p);
}

template <int EPI>
static void launch_simt(const GemmParams& p, bool ak, bool bk, dim3 grid, hipStream_t s) {
  if (ak && bk) gemm_simt_kernel<true, true, EPI><<<grid, 256, 0, s>>>(p);
  else if (ak) gemm_simt_kernel<true, false, EPI><<<grid, 256, 0, s>>>(p);
  else if (bk) gemm_simt_kernel<false, true, EPI><<<grid, 256, 0, s>>>(p);
  else gemm_simt_kernel<false, false, EPI><<<grid, 256, 0, s>>>(p);
}

int gemm_splits(int M, int N, int K, int dtype) {
  const int t = dtype == 0 ? 256 : 64;
  const long tiles = (long)((M + t - 1) / t) * ((N + t - 1) / t);
  if (tiles >= 512 || K < 2048) return 1;
  int s = (int)((1024 + tiles - 1) / tiles);
  const int maxs = K / 1024;
  if (s > maxs) s = maxs;
  if (s > 32) s = 32;
  return s < 1 ? 1 : s;
}

uint64_t gemm_ws_bytes(int M, int N, int K, int dtype) {
  const int s = gemm_splits(M, N, K, dtype);
  return s > 1 ? (uint64_t)s * M * N * 4 : 0;
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
  int splits = 1;
  if (g.epi == EPI_F32 && g.splitk_ws) splits = gemm_splits(g.M, g.N, g.K, g.dtype);
  int kchunk = g.K;
  if (splits > 1) {
    kchunk = ((g.K + splits - 1) / splits + kBK - 1) / kBK * kBK;
    splits = (g.K + kchunk - 1) / kchunk;
  }
  if (splits > 1) {
    p.e.c32 = g.splitk_ws;
    p.e.ldc = g.N;
    p.e.beta = 0;
    p.e.split_stride = (long)g.M * g.N;
  }
  p.kchunk = kchunk > 0 ? kchunk : 1;
  dim3 grid(p.tiles_m * p.tiles_n, 1, splits);
  // K == 0 runs the kernels with an empty k-loop: the epilogue sees zeros.
  if (g.dtype == 0) {
    switch (g.epi) {
      case EPI_F32: launch_mfma<EPI_F32>(p, g.a_k, g.b_k, grid, s); break;
      case EPI_RESID: launch_mfma<EPI_RESID>(p, g.a_k, g.b_k, grid, s); break;
      case EPI_LP: launch_mfma<EPI_LP>(p, g.a_k, g.b_k, grid, s); break;
      case EPI_RELU2: launch_mfma<EPI_RELU2>(p, g.a_k, g.b_k, grid, s); break;
      case EPI_DRELU2: launch_mfma<EPI_DRELU2>(p, g.a_k, g.b_k, grid, s); break;
      default: return 8;
    }
  } else {
    switch (g.epi) {
      case EPI_F32: launch_simt<EPI_F32>(p, g.a_k, g.b_k, grid, s); break;
      case EPI_RESID: launch_simt<EPI_RESID>(p, g.a_k, g.b_k, grid, s); break;
      case EPI_LP: launch_simt<EPI_LP>(p, g.a_k, g.b_k, grid, s); break;
      case EPI_RELU2: launch_simt<EPI_RELU2>(p, g.a_k, g.b_k, grid, s); break;
      case EPI_DRELU2: launch_simt<EPI_DRELU2>(p, g.a_k, g.b_k, grid, s); break;
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
