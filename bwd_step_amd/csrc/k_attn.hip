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
#include "common.h"
#include "kernels.h"

namespace nc {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

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

// ------------------------------------------------------------------ forward
template <int HD>
__global__ void __launch_bounds__(256) attn_fwd_mfma(AttnArgs p) {
  constexpr int KS = HD / 16, HB = HD / 32;
  __shared__ __attribute__((aligned(16))) bf16 Ks[64 * (HD + 8)];
  __shared__ __attribute__((aligned(16))) bf16 Vt[HD * (64 + 4)];

  const int T = p.T;
  const int nqb = (T + 127) / 128;
  const int qb = nqb - 1 - blockIdx.x;
  const int bh = blockIdx.y, b = bh / p.H, h = bh % p.H;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 5, li = lane & 31;
  const int q0 = qb * 128;
  const int qi = q0 + wv * 32 + li;
  const size_t tok0 = (size_t)b * T;

  const bf16* qp = (const bf16*)p.q + tok0 * p.ldq + h * HD;
  const bf16* kp = (const bf16*)p.k + tok0 * p.ldk + h * HD;
  const bf16* vp = (const bf16*)p.v + tok0 * p.ldv + h * HD;

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
  if (g == 0) p.lse[(size_t)bh * T + qi] = (mx + log2f(ltot)) * kLn2;
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
  const bf16* kp = (const bf16*)p.k + tok0 * p.ldk + h * HD;
  const bf16* vp = (const bf16*)p.v + tok0 * p.ldv + h * HD;
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
      lse_s[threadIdx.x] = t < T ? lsep[t] * kLog2e : 0.f;
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
  const int nqb = (T + 127) / 128;
  const int qb = nqb - 1 - blockIdx.x;
  const int bh = blockIdx.y, b = bh / p.H, h = bh % p.H;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 5, li = lane & 31;
  const int q0 = qb * 128;
  const int qi = q0 + wv * 32 + li;
  const size_t tok0 = (size_t)b * T;

  const bf16* qp = (const bf16*)p.q + tok0 * p.ldq + h * HD;
  const bf16* kp = (const bf16*)p.k + tok0 * p.ldk + h * HD;
  const bf16* vp = (const bf16*)p.v + tok0 * p.ldv + h * HD;
  const bf16* dop = (const bf16*)p.dout + tok0 * p.lddo + h * HD;

  bf16x8 qf[KS], df[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    qf[s] = qi < T ? *reinterpret_cast<const bf16x8*>(qp + (size_t)qi * p.ldq + s * 16 + g * 8) : bf16x8{};
    df[s] = qi < T ? *reinterpret_cast<const bf16x8*>(dop + (size_t)qi * p.lddo + s * 16 + g * 8) : bf16x8{};
  }
  const float lse_l = qi < T ? p.lse[(size_t)bh * T + qi] * kLog2e : 0.f;
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
    const T* kr = (const T*)p.k + (tok0 + j) * p.ldk + h * hd;
    const T* vr = (const T*)p.v + (tok0 + j) * p.ldv + h * hd;
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
    const T* kr = (const T*)p.k + (tok0 + j) * p.ldk + h * hd;
    const T* vr = (const T*)p.v + (tok0 + j) * p.ldv + h * hd;
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
  const T* kr = (const T*)p.k + (tok0 + kj) * p.ldk + h * hd;
  const T* vr = (const T*)p.v + (tok0 + kj) * p.ldv + h * hd;
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
    if (hd == 128) attn_fwd_mfma<128><<<grid, 256, 0, s>>>(p);
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
    attn_bwd_pre<bf16><<<(unsigned)((rows + 3) / 4), 256, 0, s>>>(p, hd);
    dim3 gk((p.T + 127) / 128, p.B * p.H);
    dim3 gq((p.T + 127) / 128, p.B * p.H);
    if (hd == 128) {
      attn_bwd_dkdv_mfma<128><<<gk, 256, 0, s>>>(p);
      attn_bwd_dq_mfma<128><<<gq, 256, 0, s>>>(p);
    } else if (hd == 64) {
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

}  // namespace nc
