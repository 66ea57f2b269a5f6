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
  int M, N, K;
  int kchunk;  // K range per split (multiple of 64)
  int tiles_m, tiles_n;
  EpiArgs e;
};

// ------------------------------------------------------------------ epilogue
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

// LDS element offset of the 16-byte chunk `kc` (0..7) of tile row `row`.
__device__ __forceinline__ int swz(int row, int kc) { return row * 64 + ((kc ^ (row & 7)) << 3); }

template <int ROWS, bool KMAJ>
struct TileLoader {
  // ROWS x 64 bf16 per tile = ROWS*8 chunks of 16 B; ROWS/32 per thread.
  static constexpr int NC = ROWS / 32;
  u32x4 r[NC];

  __device__ __forceinline__ void load(const bf16* __restrict__ g, long ld, int row0, int k0, int rows_lim,
                                       int k_lim) {
    const int t = threadIdx.x;
    if constexpr (KMAJ) {
#pragma unroll
      for (int q = 0; q < NC; ++q) {
        const int c = t + 256 * q;
        const int row = c >> 3, kc = c & 7;
        const int gr = row0 + row, gk = k0 + kc * 8;
        if (gr < rows_lim && gk < k_lim)
          r[q] = *reinterpret_cast<const u32x4*>(g + (size_t)gr * ld + gk);
        else
          r[q] = u32x4{0, 0, 0, 0};
      }
    } else {
      // thread owns NC consecutive k-rows of one 8-wide chunk of tile rows
      constexpr int MCH = ROWS / 8;  // chunks along the contiguous dim
      const int mc = t % MCH, kg = t / MCH;
      const int gm = row0 + mc * 8;
#pragma unroll
      for (int q = 0; q < NC; ++q) {
        const int gk = k0 + kg * NC + q;
        if (gm < rows_lim && gk < k_lim)
          r[q] = *reinterpret_cast<const u32x4*>(g + (size_t)gk * ld + gm);
        else
          r[q] = u32x4{0, 0, 0, 0};
      }
    }
  }

  __device__ __forceinline__ void store(bf16* __restrict__ s) {
    const int t = threadIdx.x;
    if constexpr (KMAJ) {
#pragma unroll
      for (int q = 0; q < NC; ++q) {
        const int c = t + 256 * q;
        const int row = c >> 3, kc = c & 7;
        *reinterpret_cast<u32x4*>(s + swz(row, kc)) = r[q];
      }
    } else {
      constexpr int MCH = ROWS / 8;
      const int mc = t % MCH, kg = t / MCH;
#pragma unroll
      for (int mm = 0; mm < 8; ++mm) {
        const uint32_t sel = (mm & 1) ? 0x07060302u : 0x05040100u;
        const int w = mm >> 1;
        const int row = mc * 8 + mm;
        if constexpr (NC == 8) {
          u32x4 o;
          o.x = __builtin_amdgcn_perm(r[1][w], r[0][w], sel);
          o.y = __builtin_amdgcn_perm(r[3][w], r[2][w], sel);
          o.z = __builtin_amdgcn_perm(r[5][w], r[4][w], sel);
          o.w = __builtin_amdgcn_perm(r[7][w], r[6][w], sel);
          *reinterpret_cast<u32x4*>(s + swz(row, kg)) = o;
        } else {
          static_assert(NC == 4, "tile rows must be 128 or 256");
          u32x2 o;
          o.x = __builtin_amdgcn_perm(r[1][w], r[0][w], sel);
          o.y = __builtin_amdgcn_perm(r[3][w], r[2][w], sel);
          *reinterpret_cast<u32x2*>(s + swz(row, kg >> 1) + ((kg & 1) << 2)) = o;
        }
      }
    }
  }
};

template <int BM, int BN, bool AK, bool BKM, int EPI>
__global__ void __launch_bounds__(256, 1) gemm_mfma_kernel(GemmParams p) {
  constexpr int WM = 2, WN = 2;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  __shared__ __attribute__((aligned(16))) bf16 As[2][BM * kBK];
  __shared__ __attribute__((aligned(16))) bf16 Bs[2][BN * kBK];

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

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int wm = wv / WN, wn = wv % WN;

  f32x16 acc[FM][FN];
#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int c = 0; c < FN; ++c) acc[a][c] = f32x16{};

  TileLoader<BM, AK> la;
  TileLoader<BN, BKM> lb;
  const bf16* Ag = (const bf16*)p.A;
  const bf16* Bg = (const bf16*)p.B;

  if (nk > 0) {
    la.load(Ag, p.lda, m0, kbeg, p.M, kend);
    lb.load(Bg, p.ldb, n0, kbeg, p.N, kend);
    la.store(As[0]);
    lb.store(Bs[0]);
  }
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      la.load(Ag, p.lda, m0, kbeg + (kt + 1) * kBK, p.M, kend);
      lb.load(Bg, p.ldb, n0, kbeg + (kt + 1) * kBK, p.N, kend);
    }
    const bf16* as = As[cur];
    const bf16* bs = Bs[cur];
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      const int kc = s * 2 + (lane >> 5);
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int a = 0; a < FM; ++a) {
        const int row = wm * TM + a * 32 + (lane & 31);
        af[a] = *reinterpret_cast<const bf16x8*>(as + swz(row, kc));
      }
#pragma unroll
      for (int c = 0; c < FN; ++c) {
        const int row = wn * TN + c * 32 + (lane & 31);
        bfr[c] = *reinterpret_cast<const bf16x8*>(bs + swz(row, kc));
      }
#pragma unroll
      for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int c = 0; c < FN; ++c)
          acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bfr[c], acc[a][c], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      la.store(As[cur ^ 1]);
      lb.store(Bs[cur ^ 1]);
    }
    __syncthreads();
  }

  // Epilogue.  Lane holds column (lane & 31) and rows 8*(r/4) + 4*(lane/32) + r%4.
#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int c = 0; c < FN; ++c) {
      const long j = n0 + wn * TN + c * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const long i = m0 + wm * TM + a * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (i < p.M && j < p.N) epi_apply<EPI, bf16>(p.e, split, i, j, acc[a][c][r]);
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
  if (ak && bk) gemm_mfma_kernel<256, 256, true, true, EPI><<<grid, 256, 0, s>>>(p);
  else if (ak) gemm_mfma_kernel<256, 256, true, false, EPI><<<grid, 256, 0, s>>>(p);
  else if (bk) gemm_mfma_kernel<256, 256, false, true, EPI><<<grid, 256, 0, s>>>(p);
  else gemm_mfma_kernel<256, 256, false, false, EPI><<<grid, 256, 0, s>>>(p);
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
