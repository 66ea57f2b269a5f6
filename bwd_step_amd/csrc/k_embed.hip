// Token embedding gather and its atomic-free backward ("nanochat explainer",
// Modern architecture choices: untied embeddings).
//
// Forward: x[n] = E[tok[n]] (fp32 residual stream).  Ids outside [0, V) set
// the status bit and are clamped so that no access leaves E.
//
// Backward: dE[v] = sum over positions n with tok[n] == v of dx[n], summed in
// increasing n, with no floating-point atomics, so the result is bitwise
// reproducible.  Steps:
//   1. a stable LSD radix sort (8-bit digits) of (id, position) pairs; each
//      pass is a per-tile digit histogram, an exclusive scan (per digit over
//      the tiles, plus each digit's base), and a stable scatter whose in-tile
//      ranks come from wavefront ballots;
//   2. the sorted positions are cut into pieces of kPiece entries; each piece
//      sums dx over every run of equal ids inside it, in order, and stores the
//      run's sum at the run's first sorted index; the first sorted index of
//      every id, lo[v] (lo[V] = N), is written from the sorted ids;
//   3. each vocabulary row takes its segment [lo[v], lo[v + 1]) and adds the
//      partial sums that start at lo and at every piece boundary inside it.
// Long segments (skewed ids) are thus split over many pieces and reduced in a
// fixed order.
#include "common.h"
#include "kernels.h"

namespace nc {

constexpr int kSortTile = 256;  // elements per radix-sort tile (one per thread)
constexpr int kPiece = 16;      // sorted entries per partial-sum piece

// --------------------------------------------------------------- forward
template <class T>
__global__ void __launch_bounds__(256) embed_fwd_kernel(const T* __restrict__ E, const int32_t* __restrict__ tok,
                                                        float* __restrict__ x, int N, int d, int V,
                                                        int* __restrict__ status) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= N) return;
  int t = tok[row];
  if (t < 0 || t >= V) {
    if (lane == 0) atomicOr(status, kStatusTokenRange);
    t = t < 0 ? 0 : V - 1;
  }
  const T* src = E + (size_t)t * d;
  float* dst = x + (size_t)row * d;
  for (int c = lane * 4; c < d; c += 256) {
    f32x4 v;
    if constexpr (sizeof(T) == 2) {
      u32x2 w = *reinterpret_cast<const u32x2*>(src + c);
      v = f32x4{bf16lo_to_f32(w.x), bf16hi_to_f32(w.x), bf16lo_to_f32(w.y), bf16hi_to_f32(w.y)};
    } else {
      v = *reinterpret_cast<const f32x4*>(src + c);
    }
    *reinterpret_cast<f32x4*>(dst + c) = v;
  }
}

int launch_embed_fwd(const void* E, const int32_t* tok, float* x, int N, int d, int V, int dtype, int* status,
                     hipStream_t s) {
  if (N == 0) return 0;
  if (dtype == 0)
    embed_fwd_kernel<bf16><<<(N + 3) / 4, 256, 0, s>>>((const bf16*)E, tok, x, N, d, V, status);
  else
    embed_fwd_kernel<float><<<(N + 3) / 4, 256, 0, s>>>((const float*)E, tok, x, N, d, V, status);
  NC_LAUNCH_CHECK();
  return 0;
}

// --------------------------------------------------------------- radix sort
// Stable rank of this thread's digit among the tile's elements with the same
// digit, and (for lane-0-of-group) the per-wave digit counts in LDS.
__device__ __forceinline__ int tile_rank(int digit, bool valid, int* cnt /*[4][256]*/, int* tot /*[256]*/) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 4 * 256; i += 256) cnt[i] = 0;
  __syncthreads();
  uint64_t peers = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const uint64_t bal = __ballot((digit >> b) & 1);
    peers &= ((digit >> b) & 1) ? bal : ~bal;
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int wrank = __popcll(peers & below);
  if (valid && wrank == 0) cnt[wv * 256 + digit] = __popcll(peers);
  __syncthreads();
  // prefix over waves for this digit
  int pre = 0;
  for (int w = 0; w < wv; ++w) pre += cnt[w * 256 + digit];
  if (tot) {
    for (int dg = threadIdx.x; dg < 256; dg += 256)
      tot[dg] = cnt[dg] + cnt[256 + dg] + cnt[512 + dg] + cnt[768 + dg];
  }
  return pre + wrank;
}

__global__ void __launch_bounds__(256) sort_hist_kernel(const int32_t* __restrict__ keys, const int32_t* __restrict__ tok,
                                                        int N, int V, int shift, int* __restrict__ hist, int ntiles) {
  __shared__ int cnt[4 * 256];
  __shared__ int tot[256];
  const int idx = blockIdx.x * kSortTile + threadIdx.x;
  const bool valid = idx < N;
  int key = 0;
  if (valid) {
    if (keys) {
      key = keys[idx];
    } else {
      key = tok[idx];
      key = key < 0 ? 0 : (key >= V ? V - 1 : key);
    }
  }
  const int digit = (key >> shift) & 255;
  tile_rank(digit, valid, cnt, tot);
  __syncthreads();
  hist[threadIdx.x * ntiles + blockIdx.x] = tot[threadIdx.x];
}

// Offsets of the scatter from the per-tile digit counts hist[digit][tile]:
// in place, hist[d][t] becomes the count of digit d in tiles before t, and
// base[d] the count of all digits below d.  One block of 16 wavefronts; a
// wavefront scans whole digit rows (four consecutive counts per lane, so the
// loads are coalesced), then one wavefront scans the 256 digit totals.
__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(x, off, 64);
    if (lane >= off) x += t;
  }
  return x;
}
__global__ void __launch_bounds__(1024) scan_kernel(int* __restrict__ hist, int ntiles, int* __restrict__ base) {
  __shared__ int tot[256];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int d = wv; d < 256; d += 16) {
    int* row = hist + (size_t)d * ntiles;
    int run = 0;
    for (int c0 = 0; c0 < ntiles; c0 += 256) {
      int v[4];
      int sum = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = c0 + 4 * lane + e;
        v[e] = i < ntiles ? row[i] : 0;
        sum += v[e];
      }
      const int incl = wave_incl_scan(sum, lane);
      int ex = run + incl - sum;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = c0 + 4 * lane + e;
        if (i < ntiles) row[i] = ex;
        ex += v[e];
      }
      run += __shfl(incl, 63, 64);
    }
    if (lane == 0) tot[d] = run;
  }
  __syncthreads();
  if (wv == 0) {
    int v[4];
    int sum = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = tot[4 * lane + e];
      sum += v[e];
    }
    int ex = wave_incl_scan(sum, lane) - sum;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      base[4 * lane + e] = ex;
      ex += v[e];
    }
  }
}

__global__ void __launch_bounds__(256) sort_scatter_kernel(const int32_t* __restrict__ keys_in,
                                                           const int32_t* __restrict__ vals_in,
                                                           const int32_t* __restrict__ tok, int N, int V, int shift,
                                                           const int* __restrict__ offs,
                                                           const int* __restrict__ base, int ntiles,
                                                           int32_t* __restrict__ keys_out,
                                                           int32_t* __restrict__ vals_out) {
  __shared__ int cnt[4 * 256];
  const int idx = blockIdx.x * kSortTile + threadIdx.x;
  const bool valid = idx < N;
  int key = 0, val = idx;
  if (valid) {
    if (keys_in) {
      key = keys_in[idx];
      val = vals_in[idx];
    } else {
      key = tok[idx];
      key = key < 0 ? 0 : (key >= V ? V - 1 : key);
    }
  }
  const int digit = (key >> shift) & 255;
  const int rank = tile_rank(digit, valid, cnt, nullptr);
  if (valid) {
    const int dst = base[digit] + offs[digit * ntiles + blockIdx.x] + rank;
    keys_out[dst] = key;
    vals_out[dst] = val;
  }
}

// --------------------------------------------------------------- run sums
// Block per piece of kPiece sorted entries; threads stride over columns.
__global__ void __launch_bounds__(256) piece_sum_kernel(const float* __restrict__ dx, const int32_t* __restrict__ skey,
                                                        const int32_t* __restrict__ spos, int N, int d,
                                                        float* __restrict__ partial) {
  const int p0 = blockIdx.x * kPiece;
  const int p1 = min(p0 + kPiece, N);
  __shared__ int k_s[kPiece], pos_s[kPiece];
  if (threadIdx.x < kPiece && p0 + (int)threadIdx.x < N) {
    k_s[threadIdx.x] = skey[p0 + threadIdx.x];
    pos_s[threadIdx.x] = spos[p0 + threadIdx.x];
  }
  __syncthreads();
  for (int c = threadIdx.x * 4; c < d; c += 1024) {
    f32x4 acc = *reinterpret_cast<const f32x4*>(dx + (size_t)pos_s[0] * d + c);
    int start = p0;
    for (int e = p0 + 1; e < p1; ++e) {
      const int le = e - p0;
      if (k_s[le] != k_s[le - 1]) {
        *reinterpret_cast<f32x4*>(partial + (size_t)start * d + c) = acc;
        start = e;
        acc = *reinterpret_cast<const f32x4*>(dx + (size_t)pos_s[le] * d + c);
      } else {
        acc += *reinterpret_cast<const f32x4*>(dx + (size_t)pos_s[le] * d + c);
      }
    }
    *reinterpret_cast<f32x4*>(partial + (size_t)start * d + c) = acc;
  }
}

// lo[v] = the first sorted index whose id is >= v, for v = 0 .. V (lo[V] =
// N): thread i (0 <= i <= N) writes every v in (id[i - 1], id[i]] (with
// id[-1] = -1, id[N] = V), so each v is written exactly once.
__global__ void __launch_bounds__(256) seg_lo_kernel(const int32_t* __restrict__ skey, int N, int V,
                                                     int32_t* __restrict__ lo) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i > N) return;
  const int a = i == 0 ? -1 : skey[i - 1];
  const int b = i == N ? V : skey[i];
  for (int v = a + 1; v <= b; ++v) lo[v] = i;
}

// Wavefront per vocabulary row.
__global__ void __launch_bounds__(256) row_combine_kernel(const float* __restrict__ partial,
                                                          const int32_t* __restrict__ seg_lo, int d, int V,
                                                          float* __restrict__ dE, int accumulate) {
  const int v = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (v >= V) return;
  const int lo = seg_lo ? seg_lo[v] : 0;
  const int hi = seg_lo ? seg_lo[v + 1] : 0;
  float* dst = dE + (size_t)v * d;
  for (int c = lane * 4; c < d; c += 256) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (lo < hi) {
      acc = *reinterpret_cast<const f32x4*>(partial + (size_t)lo * d + c);
      for (int p = (lo / kPiece + 1) * kPiece; p < hi; p += kPiece)
        acc += *reinterpret_cast<const f32x4*>(partial + (size_t)p * d + c);
    }
    if (accumulate) {
      if (lo < hi) *reinterpret_cast<f32x4*>(dst + c) += acc;
    } else {
      *reinterpret_cast<f32x4*>(dst + c) = acc;
    }
  }
}

static inline size_t al256(size_t b) { return (b + 255) & ~(size_t)255; }

uint64_t embed_bwd_ws_bytes(int N, int d, int V) {
  const int ntiles = (N + kSortTile - 1) / kSortTile;
  return 4 * al256((size_t)N * 4) + al256((size_t)256 * ntiles * 4) + al256(256 * 4) + al256(((size_t)V + 1) * 4) +
         al256((size_t)N * d * 4);
}

int launch_embed_bwd(const float* dx, const int32_t* tok, float* dE, int N, int d, int V, int accumulate, void* ws,
                     hipStream_t s) {
  if (V == 0) return 0;
  const int ntiles = (N + kSortTile - 1) / kSortTile;
  char* p = (char*)ws;
  int32_t* ka = (int32_t*)p; p += al256((size_t)N * 4);
  int32_t* va = (int32_t*)p; p += al256((size_t)N * 4);
  int32_t* kb = (int32_t*)p; p += al256((size_t)N * 4);
  int32_t* vb = (int32_t*)p; p += al256((size_t)N * 4);
  int* hist = (int*)p; p += al256((size_t)256 * ntiles * 4);
  int* base = (int*)p; p += al256(256 * 4);
  int32_t* seg_lo = (int32_t*)p; p += al256(((size_t)V + 1) * 4);
  float* partial = (float*)p;
  if (N > 0) {
    int bits = 1;
    while ((1 << bits) < V) ++bits;
    const int passes = (bits + 7) / 8;
    const int32_t* kin = nullptr;
    const int32_t* vin = nullptr;
    int32_t* kout = ka;
    int32_t* vout = va;
    for (int ps = 0; ps < passes; ++ps) {
      sort_hist_kernel<<<ntiles, 256, 0, s>>>(kin, tok, N, V, 8 * ps, hist, ntiles);
      scan_kernel<<<1, 1024, 0, s>>>(hist, ntiles, base);
      sort_scatter_kernel<<<ntiles, 256, 0, s>>>(kin, vin, tok, N, V, 8 * ps, hist, base, ntiles, kout, vout);
      kin = kout;
      vin = vout;
      kout = (kout == ka) ? kb : ka;
      vout = (vout == va) ? vb : va;
    }
    piece_sum_kernel<<<(N + kPiece - 1) / kPiece, 256, 0, s>>>(dx, kin, vin, N, d, partial);
    seg_lo_kernel<<<(N + 1 + 255) / 256, 256, 0, s>>>(kin, N, V, seg_lo);
    row_combine_kernel<<<(V + 3) / 4, 256, 0, s>>>(partial, seg_lo, d, V, dE, accumulate);
  } else if (!accumulate) {
    // no tokens: every row is absent
    row_combine_kernel<<<(V + 3) / 4, 256, 0, s>>>(nullptr, nullptr, d, V, dE, 0);
  }
  NC_LAUNCH_CHECK();
  return 0;
}

}  // namespace nc
