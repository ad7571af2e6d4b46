// route.hip — router scores, softmax top-k, expert histogram, scan and the
// stable expert-major permutation; routing backward and router wgrad.
//
// Pages: a router scores each token, the top-k experts are chosen and the
// choice becomes a permutation index ([P2] 1.1, 2.1); the routing metadata
// stays resident on the GPU ([P1] 核心特点 二, GPU-resident routing).
//
// Device layout of the routing workspace: block_counts[E][nblk] int32 with
// nblk = ceil(T / 64) (one block of 64 tokens each): expert-major, so the scan kernel reads each expert's
// per-block counts contiguously.
#include <hip/hip_runtime.h>

#include <mutex>

#include "common.h"

using namespace moe;

namespace {

constexpr int kTokBlock = 64;  // tokens per routing block (one wave, one token per lane)

// ---------------------------------------------------------------- scores
// Small-E router scores on the vector ALUs: one wave per token at a time; each
// lane takes 16-byte chunks of the token's row and the matching rows of W_r
// (E contiguous values per feature), accumulating all E dot products in
// registers; the E partial sums are reduced across the wave in a fixed order.
// One launch covers the experts [e0, e0 + Ec) with Ec <= EMAX; E is the row
// length of W_r and of the logits.  (bf16 with E > 16 and E % 8 == 0 uses the
// MFMA grouped GEMM with a single group, see gemm_bf16.hip; any other E above
// 64 runs here as several 64-expert launches, each reading x again.)
template <typename T, int EMAX, bool EXACT>
__global__ void __launch_bounds__(256) router_logits_small_kernel(const T* __restrict__ x,
                                                                  const T* __restrict__ wr, int T_,
                                                                  int d, int E, int e0, int Ec,
                                                                  float* __restrict__ logits) {
  constexpr int V = 16 / sizeof(T);
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int nwaves = (gridDim.x * blockDim.x) >> 6;
  const int nchunk = d / V;
  float acc[EMAX];
  for (int t = wave; t < T_; t += nwaves) {
#pragma unroll
    for (int e = 0; e < EMAX; ++e) acc[e] = 0.f;
    const T* xr = x + (size_t)t * d;
    for (int c = lane; c < nchunk; c += 64) {
      const uint4 xraw = *reinterpret_cast<const uint4*>(xr + (size_t)c * V);
      const T* xv = reinterpret_cast<const T*>(&xraw);
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const float xf = Elem<T>::ld(xv, v);
        const T* wrow = wr + (size_t)(c * V + v) * E + e0;
        if constexpr (EXACT) {
          constexpr int NV = EMAX * sizeof(T) / 16;
#pragma unroll
          for (int q = 0; q < NV; ++q) {
            const uint4 wraw = *reinterpret_cast<const uint4*>(wrow + q * V);
            const T* wv = reinterpret_cast<const T*>(&wraw);
#pragma unroll
            for (int i = 0; i < V; ++i) acc[q * V + i] += xf * Elem<T>::ld(wv, i);
          }
        } else {
#pragma unroll
          for (int e = 0; e < EMAX; ++e)
            if (e < Ec) acc[e] += xf * Elem<T>::ld(wrow, e);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      float v = acc[e];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
      acc[e] = v;
    }
    if (lane == 0) {
#pragma unroll
      for (int e = 0; e < EMAX; ++e)
        if (e < Ec) logits[(size_t)t * E + e0 + e] = acc[e];
    }
  }
}

// ---------------------------------------------------------------- top-k
// A block takes 64 tokens with LPT lanes per token (4, 8 or 16 by expert
// count).  The block's logits are staged in LDS a chunk of experts at a time
// (coalesced loads, sixteen in flight per thread; the odd row pitch spreads
// the column walks over the banks).  Each lane keeps a sorted list of its
// 1/LPT share of every chunk: experts are visited in ascending index, a
// candidate enters only if its logit is strictly larger than the k-th kept
// one and lands behind every kept expert with an equal or larger logit, so
// each list is ordered by (logit descending, index ascending).  The LPT
// lists are then merged with k rounds of a shuffle reduction under the same
// order.  NaN scores count as
// -inf.  Gates are the softmax over the k kept logits.  The block also counts
// its tokens' experts in LDS and writes its histogram column to the workspace.
constexpr int kTopkChunk = 128;   // experts staged per pass
template <int KMAX, int LPT>
__global__ void __launch_bounds__(64 * LPT) topk_hist_kernel(
    const float* __restrict__ logits, int T_, int E, int k, int32_t* __restrict__ topk_idx,
    float* __restrict__ gates, int32_t* __restrict__ block_counts, int nblk) {
  constexpr int kTopkThreads = 64 * LPT;  // LPT lanes per token
  __shared__ float stage[kTokBlock * (kTopkChunk + 1)];
  __shared__ int hist[1024];
  const int tid = threadIdx.x;
  const int tl = tid / LPT, sub = tid % LPT;
  for (int e = tid; e < E; e += kTopkThreads) hist[e] = 0;
  const int tbase = blockIdx.x * kTokBlock;
  const int ntok = min(kTokBlock, T_ - tbase);
  float val[KMAX];
  int idx[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    val[i] = -INFINITY;
    idx[i] = -1;
  }
  for (int c0 = 0; c0 < E; c0 += kTopkChunk) {
    const int ce = min(kTopkChunk, E - c0);
    __syncthreads();  // the previous chunk has been consumed
    // element i of the [ntok][ce] chunk goes to stage[r][c]
    const int n = ntok * ce;
    const float inv_ce = 1.0f / (float)ce;
    for (int base = 0; base < n; base += 16 * kTopkThreads) {
      float v[16];
      int pos[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int i = base + j * kTopkThreads + tid;
        int r = (int)((float)i * inv_ce);
        int c = i - r * ce;
        if (c < 0) {
          --r;
          c += ce;
        } else if (c >= ce) {
          ++r;
          c -= ce;
        }
        pos[j] = i < n ? r * (kTopkChunk + 1) + c : -1;
        v[j] = i < n ? logits[(size_t)(tbase + r) * E + c0 + c] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (pos[j] >= 0) stage[pos[j]] = v[j];
    }
    __syncthreads();
    if (tl < ntok) {
      const int q = (ce + LPT - 1) / LPT;
      const int lo = sub * q, hi = min(lo + q, ce);
      const float* row = stage + tl * (kTopkChunk + 1);
      for (int c = lo; c < hi; ++c) {
        float v = row[c];
        if (v != v) v = -INFINITY;
        // position = number of kept experts that stay ahead of this one
        int p = 0;
#pragma unroll
        for (int i = 0; i < KMAX; ++i)
          if (i < k) p += (idx[i] >= 0 && val[i] >= v) ? 1 : 0;
        if (p < k) {
#pragma unroll
          for (int i = KMAX - 1; i > 0; --i) {
            if (i < k && i > p) {
              val[i] = val[i - 1];
              idx[i] = idx[i - 1];
            }
          }
#pragma unroll
          for (int i = 0; i < KMAX; ++i) {
            if (i == p) {
              val[i] = v;
              idx[i] = c0 + c;
            }
          }
        }
      }
    }
  }
  // merge the LPT lists: k rounds, each taking the best head of the LPT
  float mv[KMAX];
  int mi[KMAX];
  int h = 0;  // next entry of this lane's own list
#pragma unroll
  for (int r = 0; r < KMAX; ++r) {
    mv[r] = -INFINITY;
    mi[r] = -1;
    if (r < k) {
      float bv = -INFINITY;
      int bi = -1;
#pragma unroll
      for (int i = 0; i < KMAX; ++i)
        if (i == h) {
          bv = val[i];
          bi = idx[i];
        }
      int bs = sub;
#pragma unroll
      for (int off = 1; off < LPT; off <<= 1) {
        const float ov = __shfl_xor(bv, off, LPT);
        const int oi = __shfl_xor(bi, off, LPT);
        const int os = __shfl_xor(bs, off, LPT);
        // (ov, oi) precedes (bv, bi): larger logit, then lower index; empty last
        const bool take = oi >= 0 && (bi < 0 || ov > bv || (ov == bv && oi < bi));
        if (take) {
          bv = ov;
          bi = oi;
          bs = os;
        }
      }
      mv[r] = bv;
      mi[r] = bi;
      if (bs == sub) ++h;
    }
  }
  if (tl < ntok && sub == 0) {
    const int t = tbase + tl;
    // softmax over the kept logits (mv[0] is the largest)
    const float m = mv[0];
    float z = 0.f;
    float ex[KMAX];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      ex[i] = (i < k) ? expf(mv[i] - m) : 0.f;
      z += ex[i];
    }
    const float inv = 1.0f / z;
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      if (i < k) {
        topk_idx[(size_t)t * k + i] = mi[i];
        gates[(size_t)t * k + i] = ex[i] * inv;
        atomicAdd(&hist[mi[i]], 1);
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kTopkThreads)
    block_counts[(size_t)e * nblk + blockIdx.x] = hist[e];
}

// Block-wide exclusive scan of one int per thread (blockDim.x == 256).
__device__ int block_exclusive_scan(int v, int* sh /*[256]*/, int* total) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    int add = tid >= off ? sh[tid - off] : 0;
    __syncthreads();
    sh[tid] += add;
    __syncthreads();
  }
  int incl = sh[tid];
  if (total) *total = sh[255];
  __syncthreads();
  return incl - v;
}

// One block per expert: exclusive scan of the expert's per-block counts (in
// place: block_counts becomes each block's base row inside the expert) and the
// expert's total count.
__global__ void __launch_bounds__(256) expert_scan_kernel(int32_t* __restrict__ block_counts,
                                                          int nblk, int32_t* __restrict__ counts) {
  __shared__ int sh[256];
  const int e = blockIdx.x;
  int32_t* col = block_counts + (size_t)e * nblk;
  const int per = (nblk + 255) / 256;
  const int b0 = threadIdx.x * per;
  int local = 0;
  for (int i = 0; i < per; ++i)
    if (b0 + i < nblk) local += col[b0 + i];
  int total;
  int run = block_exclusive_scan(local, sh, &total);
  for (int i = 0; i < per; ++i) {
    if (b0 + i < nblk) {
      int c = col[b0 + i];
      col[b0 + i] = run;
      run += c;
    }
  }
  if (threadIdx.x == 0) counts[e] = total;
}

// Offsets (exclusive scan over experts, recomputed by every block from the
// counts with a wave scan) and the stable ranks: the row of (t,j) with
// e = topk[t,j] is offsets[e] + (rows of e in earlier blocks) + (earlier
// tokens of this block that chose e).  Experts within a token are distinct,
// so the earlier tokens that chose e are the earlier (token, slot) pairs
// holding e.  One thread per (token, slot) pair of the block (kRankThreads
// threads, four waves on the four SIMDs), each counting over the block's
// earlier pairs read from LDS (the same address in every lane: a broadcast).
constexpr int kRankThreads = 256;
template <int KMAX>
__global__ void __launch_bounds__(kRankThreads) rank_kernel(
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ block_counts, int nblk,
    const int32_t* __restrict__ counts, int T_, int E, int k, int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_of, int32_t* __restrict__ src_tk) {
  __shared__ int offs[1025];
  __shared__ int sel[kTokBlock * KMAX];
  const int tid = threadIdx.x;
  if (tid < 64) {
    // offsets: each lane of wave 0 owns `per` consecutive experts (per <= 16)
    const int per = (E + 63) / 64;
    int local = 0;
    for (int q = 0; q < per; ++q) {
      const int e = tid * per + q;
      if (e < E) local += counts[e];
    }
    int incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (tid >= off) incl += y;
    }
    const int total = __shfl(incl, 63, 64);
    int run = incl - local;
    for (int q = 0; q < per; ++q) {
      const int e = tid * per + q;
      if (e < E) {
        offs[e] = run;
        run += counts[e];
      }
    }
    if (tid == 0) offs[E] = total;
  }
  const int tbase = blockIdx.x * kTokBlock;
  const int ntok = min(kTokBlock, T_ - tbase);
  const int npair = ntok * k;  // pairs p = t_local * k + j of this block
  for (int p = tid; p < npair; p += kRankThreads) sel[p] = topk_idx[(size_t)tbase * k + p];
  __syncthreads();
  if (blockIdx.x == 0)
    for (int e = tid; e <= E; e += kRankThreads) offsets[e] = offs[e];
  for (int p = tid; p < npair; p += kRankThreads) {
    const int tl = p / k;  // token within the block
    const int e = sel[p];
    int rank = 0;
    for (int q = 0; q < tl * k; ++q) rank += (sel[q] == e) ? 1 : 0;
    const int row = offs[e] + block_counts[(size_t)e * nblk + blockIdx.x] + rank;
    const int flat = tbase * k + p;
    row_of[flat] = row;
    src_tk[row] = flat;
  }
}

template <int KMAX>
void launch_route(const float* logits, int T_, int E, int k, int32_t* topk_idx, float* gates,
                  int32_t* counts, int32_t* offsets, int32_t* row_of, int32_t* src_tk,
                  int32_t* block_counts, int nblk, moe_ctx* ctx) {
  hipStream_t s = ctx->stream;
  {
    moe_prof_scope ps(ctx, MOE_K_TOPK);
    // lanes per token by expert count (measured on 16384-32768 tokens: E = 128
    // 19 -> 14 us with eight lanes, E = 1024 175 -> 90 us with sixteen)
    if (E > 256)
      topk_hist_kernel<KMAX, 16><<<nblk, 1024, 0, s>>>(logits, T_, E, k, topk_idx, gates, block_counts, nblk);
    else if (E > 64)
      topk_hist_kernel<KMAX, 8><<<nblk, 512, 0, s>>>(logits, T_, E, k, topk_idx, gates, block_counts, nblk);
    else
      topk_hist_kernel<KMAX, 4><<<nblk, 256, 0, s>>>(logits, T_, E, k, topk_idx, gates, block_counts, nblk);
  }
  {
    moe_prof_scope ps(ctx, MOE_K_SCAN);
    expert_scan_kernel<<<E, 256, 0, s>>>(block_counts, nblk, counts);
  }
  moe_prof_scope ps(ctx, MOE_K_RANK);
  rank_kernel<KMAX><<<nblk, kRankThreads, 0, s>>>(topk_idx, block_counts, nblk, counts, T_, E, k,
                                                  offsets, row_of, src_tk);
}

__global__ void fill_i32_kernel(int32_t* p, int n, int v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// ---------------------------------------------------------------- backward
__global__ void route_bwd_kernel(const float* __restrict__ gates, const float* __restrict__ dgates,
                                 int T_, int k, float* __restrict__ dls,
                                 const int32_t* __restrict__ row_of, float* __restrict__ dl_rows) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T_) return;
  const float* g = gates + (size_t)t * k;
  const float* dg = dgates + (size_t)t * k;
  float s = 0.f;
  for (int j = 0; j < k; ++j) s += g[j] * dg[j];
  for (int j = 0; j < k; ++j) {
    const float v = g[j] * (dg[j] - s);
    dls[(size_t)t * k + j] = v;
    if (dl_rows) dl_rows[row_of[(size_t)t * k + j]] = v;  // expert-row order
  }
}

// Router weight gradient, two passes so that a hot expert's rows spread over
// the whole chip (with skewed routing one expert can own a fifth of all
// rows).  Pass 1: the rows of every expert are cut into chunks of kRwChunk;
// one block per (64*V-feature range, chunk), V features (16 bytes) per lane,
// wave w walking the chunk's rows w, w+4, ... with eight row gathers in
// flight, fp32 sums in row order, the four waves summed in a fixed order into
// an fp32 partial per chunk.  Pass 2: dW_r[:, e] is the sum of expert e's
// chunk partials in chunk order.  Deterministic for given routing.
constexpr int kRwChunk = 256;
__host__ __device__ inline int rw_chunk_bound(int R, int E) { return R / kRwChunk + E; }

template <typename T>
__global__ void __launch_bounds__(256) router_wgrad_part_kernel(
    const T* __restrict__ x, const float* __restrict__ dls, const int32_t* __restrict__ src_tk,
    const int32_t* __restrict__ offsets, int d, int E, int k, float* __restrict__ part,
    int32_t* __restrict__ cstart) {
  constexpr int V = 16 / sizeof(T);  // features per lane
  constexpr int FC = 64 * V;         // features per block
  constexpr int U = 8;               // rows in flight per wave
  __shared__ float red[4][FC];
  __shared__ int sh[2];
  const int y = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  // expert and first row of chunk y: wave 0 scans the chunk counts
  if (w == 0) {
    const int per = (E + 63) / 64;  // <= 16 experts per lane
    int cnt[16];
    int local = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int e = lane * per + q;
      cnt[q] = (q < per && e < E) ? (offsets[e + 1] - offsets[e] + kRwChunk - 1) / kRwChunk : 0;
      local += cnt[q];
    }
    int incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off, 64);
      if (lane >= off) incl += v;
    }
    if (lane == 0) sh[0] = -1;
    int run = incl - local;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int e = lane * per + q;
      if (y == 0 && blockIdx.x == 0 && q < per && e < E) {
        cstart[e] = run;  // first chunk of each expert, for pass 2
        if (e == E - 1) cstart[E] = run + cnt[q];
      }
      if (cnt[q] > 0 && y >= run && y < run + cnt[q]) {
        sh[0] = e;
        sh[1] = offsets[e] + (y - run) * kRwChunk;
      }
      run += cnt[q];
    }
  }
  __syncthreads();
  if (sh[0] < 0) return;
  const int e = sh[0], c0 = sh[1];
  const int c1 = min(c0 + kRwChunk, offsets[e + 1]);
  const int f0 = blockIdx.x * FC;
  float acc[V];
#pragma unroll
  for (int v = 0; v < V; ++v) acc[v] = 0.f;
  const int fi = f0 + lane * V;
  if (fi < d) {  // d % 8 == 0: a lane's 16-byte chunk is wholly inside or outside
    auto add = [&](float wt, const uint4& raw) {
      const T* xv = reinterpret_cast<const T*>(&raw);
#pragma unroll
      for (int v = 0; v < V; ++v) acc[v] += wt * Elem<T>::ld(xv, v);
    };
    int r = c0 + w;
    for (; r + 4 * (U - 1) < c1; r += 4 * U) {
      int flat[U];
      float wt[U];
      uint4 raw[U];
#pragma unroll
      for (int j = 0; j < U; ++j) flat[j] = src_tk[r + 4 * j];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        wt[j] = dls[flat[j]];
        raw[j] = *reinterpret_cast<const uint4*>(x + (size_t)(flat[j] / k) * d + fi);
      }
#pragma unroll
      for (int j = 0; j < U; ++j) add(wt[j], raw[j]);
    }
    for (; r < c1; r += 4) {
      const int flat = src_tk[r];
      add(dls[flat], *reinterpret_cast<const uint4*>(x + (size_t)(flat / k) * d + fi));
    }
  }
#pragma unroll
  for (int v = 0; v < V; ++v) red[w][lane * V + v] = acc[v];
  __syncthreads();
  for (int f = threadIdx.x; f < FC; f += 256)
    if (f0 + f < d) part[(size_t)y * d + f0 + f] = ((red[0][f] + red[1][f]) + red[2][f]) + red[3][f];
}

// Pass 2: one thread per (feature, expert); no chunks (an expert without
// rows, or cstart == nullptr for an empty batch) gives exact zeros.
template <typename T>
__global__ void router_wgrad_sum_kernel(const float* __restrict__ part,
                                        const int32_t* __restrict__ cstart, int d, int E,
                                        T* __restrict__ dwr) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)d * E) return;
  const int f = (int)(i / E), e = (int)(i % E);
  float s = 0.f;
  if (cstart) {
    const int cb = cstart[e], ce = cstart[e + 1];
    for (int c = cb; c < ce; ++c) s += part[(size_t)c * d + f];
  }
  Elem<T>::st(dwr, (size_t)f * E + e, s);
}


}  // namespace

// ---------------------------------------------------------------- C ABI
using namespace moe_host;

size_t moe_internal_router_dense_ws_bytes(int T_, int d, int E);  // stats.hip
static size_t route_ws_bytes(int T_, int E) {
  const size_t nblk = (size_t)(T_ + kTokBlock - 1) / kTokBlock;
  return ((size_t)E * nblk * sizeof(int32_t) + 255) & ~(size_t)255;
}

// Routing scratch of moe_route_noalloc: block_counts of up to kScratchInts
// entries (E * ceil(T / 64) <= 2^20, 4 MiB), one copy per GPU for the life of
// the process.  Host code never uses this name as an address: it is resolved
// per device with hipGetSymbolAddress and kept in scratch_ptr.
constexpr size_t kScratchInts = (size_t)1 << 20;
static __device__ __align__(256) int32_t scratch[kScratchInts];

// Device address of `scratch` on `device`, looked up once per device with that
// device current (each GPU holds its own copy at its own address).
static moe_status scratch_address(moe_ctx* ctx, int32_t** out) {
  static std::mutex mu;
  static int32_t* scratch_ptr[64] = {nullptr};
  const int dev = ctx->device;
  if (dev < 0 || dev >= 64) return fail(ctx, MOE_ERR_UNSUPPORTED, "moe_route_noalloc: device %d", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (scratch_ptr[dev] == nullptr) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    void* ptr = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || ptr == nullptr)
      return fail(ctx, MOE_ERR_HIP, "moe_route_noalloc: scratch address on device %d: %s", dev,
                  hipGetErrorString(e));
    scratch_ptr[dev] = static_cast<int32_t*>(ptr);
  }
  *out = scratch_ptr[dev];
  return MOE_OK;
}

// Router weight-gradient partials: one fp32 row of d per row chunk, then the
// first-chunk index of every expert.
static size_t router_wgrad_ws_bytes(int T_, int d, int E, int k) {
  const size_t parts = (size_t)rw_chunk_bound(T_ * k, E) * d * sizeof(float);
  return ((parts + 255) & ~(size_t)255) + (((size_t)(E + 1) * sizeof(int32_t) + 255) & ~(size_t)255);
}

// Router-transpose scratch used by moe_permute_bwd (W_r^T, [E,d]).
size_t moe_internal_wrt_bytes(int d, int E, moe_dtype dt) {
  return ((size_t)d * E * esize(dt) + 255) & ~(size_t)255;
}

// Defined in stats.hip: workspace of the routing statistics and gradient norms.
size_t moe_internal_stats_ws_bytes(int E);

// Defined in gemm_bf16.hip: router scores through the MFMA GEMM.
moe_status moe_internal_router_logits_mfma(moe_ctx* ctx, const void* x, const void* wr, int T_,
                                           int d, int E, float* logits);

extern "C" {

moe_status moe_workspace_size(moe_ctx* ctx, int T_, int d, int E, int k, moe_dtype dtype,
                              size_t* bytes) {
  MOE_CHECK_CTX(ctx);
  MOE_REQUIRE_DTYPE(ctx, dtype);
  MOE_REQUIRE(ctx, bytes != nullptr, "bytes is null");
  MOE_REQUIRE(ctx, T_ >= 0 && d >= 8 && E >= 1 && E <= 1024 && k >= 1 && k <= E && k <= 32,
              "bad shape T=%d d=%d E=%d k=%d", T_, d, E, k);
  const size_t a = route_ws_bytes(T_, E), b = moe_internal_wrt_bytes(d, E, dtype),
               c = moe_internal_stats_ws_bytes(E), r = router_wgrad_ws_bytes(T_, d, E, k),
               dn = moe_internal_router_dense_ws_bytes(T_, d, E);
  *bytes = std::max(std::max(std::max(a, r), std::max(b, c)), dn);
  return MOE_OK;
}

moe_status moe_router_logits(moe_ctx* ctx, const void* x, const void* w_router, int T_, int d,
                             int E, moe_dtype dtype, float* logits) {
  MOE_CHECK_CTX(ctx);
  MOE_REQUIRE_DTYPE(ctx, dtype);
  MOE_REQUIRE(ctx, T_ >= 0 && d >= 8 && d % 8 == 0 && E >= 1 && E <= 1024,
              "moe_router_logits: bad shape T=%d d=%d E=%d", T_, d, E);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, x, T_ == 0);
  MOE_REQUIRE_PTR(ctx, w_router);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, logits, T_ == 0);
  if (T_ == 0) return MOE_OK;
  moe_prof_scope ps(ctx, MOE_K_ROUTER_LOGITS);
  if (dtype == MOE_BF16 && E > 16 && E % 8 == 0 && d % 64 == 0)
    return moe_internal_router_logits_mfma(ctx, x, w_router, T_, d, E, logits);
  const int blocks = std::min(1024, (T_ + 3) / 4);
#define RL_LAUNCH(TY, EM, EX)                                                                   \
  router_logits_small_kernel<TY, EM, EX><<<blocks, 256, 0, ctx->stream>>>(                      \
      (const TY*)x, (const TY*)w_router, T_, d, E, 0, E, logits)
#define RL_CASE(EM)                                                                             \
  if (E <= EM) {                                                                                \
    if (dtype == MOE_BF16) {                                                                    \
      if (E == EM && (EM * 2) % 16 == 0) RL_LAUNCH(bf16_t, EM, (EM * 2) % 16 == 0);             \
      else RL_LAUNCH(bf16_t, EM, false);                                                        \
    } else {                                                                                    \
      if (E == EM && (EM * 4) % 16 == 0) RL_LAUNCH(float, EM, (EM * 4) % 16 == 0);              \
      else RL_LAUNCH(float, EM, false);                                                         \
    }                                                                                           \
    return check_launch(ctx, "moe_router_logits");                                              \
  }
  RL_CASE(4)
  RL_CASE(8)
  RL_CASE(16)
  RL_CASE(32)
  RL_CASE(64)
#undef RL_CASE
#undef RL_LAUNCH
  // E > 64 without the MFMA path (fp32, or bf16 with E % 8 != 0): 64
  // experts per launch
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int ec = std::min(64, E - e0);
    if (dtype == MOE_BF16)
      router_logits_small_kernel<bf16_t, 64, false><<<blocks, 256, 0, ctx->stream>>>(
          (const bf16_t*)x, (const bf16_t*)w_router, T_, d, E, e0, ec, logits);
    else
      router_logits_small_kernel<float, 64, false><<<blocks, 256, 0, ctx->stream>>>(
          (const float*)x, (const float*)w_router, T_, d, E, e0, ec, logits);
  }
  return check_launch(ctx, "moe_router_logits");
}

}  // extern "C"

// Checks shared by moe_route and moe_route_noalloc.
static moe_status route_validate(moe_ctx* ctx, const float* logits, int T_, int E, int k,
                                 int32_t* topk_idx, float* gates, int32_t* counts, int32_t* offsets,
                                 int32_t* row_of, int32_t* src_tk) {
  MOE_CHECK_CTX(ctx);
  MOE_REQUIRE(ctx, T_ >= 0 && E >= 1 && E <= 1024 && k >= 1 && k <= E && k <= 32,
              "moe_route: bad shape T=%d E=%d k=%d", T_, E, k);
  MOE_REQUIRE(ctx, (int64_t)T_ * k < (int64_t)1 << 31, "moe_route: T*k >= 2^31");
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, logits, T_ == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, topk_idx, T_ == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, gates, T_ == 0);
  MOE_REQUIRE_PTR(ctx, counts);
  MOE_REQUIRE_PTR(ctx, offsets);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, row_of, T_ == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, src_tk, T_ == 0);
  {
    const size_t tk = (size_t)T_ * k * 4;
    MOE_REQUIRE_DISJOINT(ctx, "moe_route", {topk_idx, tk, "topk_idx"}, {gates, tk, "gates"},
                         {counts, (size_t)E * 4, "counts"}, {offsets, (size_t)(E + 1) * 4, "offsets"},
                         {row_of, tk, "row_of"}, {src_tk, tk, "src_tk"});
  }
  return MOE_OK;
}

// Routing with block_counts in `bc` (E * ceil(T / 64) int32, fully written by
// the top-k kernel before it is read).
static moe_status route_launch(moe_ctx* ctx, const float* logits, int T_, int E, int k,
                               int32_t* topk_idx, float* gates, int32_t* counts, int32_t* offsets,
                               int32_t* row_of, int32_t* src_tk, int32_t* bc) {
  const int nblk = (T_ + kTokBlock - 1) / kTokBlock;
  if (T_ == 0) {
    // no tokens: every count and offset is zero
    fill_i32_kernel<<<(E + 256) / 256, 256, 0, ctx->stream>>>(counts, E, 0);
    fill_i32_kernel<<<(E + 256) / 256, 256, 0, ctx->stream>>>(offsets, E + 1, 0);
    return check_launch(ctx, "moe_route");
  }
  if (k <= 2)
    launch_route<2>(logits, T_, E, k, topk_idx, gates, counts, offsets, row_of, src_tk, bc, nblk,
                    ctx);
  else if (k <= 4)
    launch_route<4>(logits, T_, E, k, topk_idx, gates, counts, offsets, row_of, src_tk, bc, nblk,
                    ctx);
  else if (k <= 8)
    launch_route<8>(logits, T_, E, k, topk_idx, gates, counts, offsets, row_of, src_tk, bc, nblk,
                    ctx);
  else
    launch_route<32>(logits, T_, E, k, topk_idx, gates, counts, offsets, row_of, src_tk, bc, nblk,
                     ctx);
  return check_launch(ctx, "moe_route");
}

extern "C" {

moe_status moe_route(moe_ctx* ctx, const float* logits, int T_, int E, int k, int32_t* topk_idx,
                     float* gates, int32_t* counts, int32_t* offsets, int32_t* row_of,
                     int32_t* src_tk) {
  moe_status st = route_validate(ctx, logits, T_, E, k, topk_idx, gates, counts, offsets, row_of, src_tk);
  if (st != MOE_OK) return st;
  const size_t need = route_ws_bytes(T_, E);
  if (ctx->ws == nullptr || ctx->ws_bytes < need)
    return fail(ctx, MOE_ERR_WORKSPACE, "moe_route: workspace %zu bytes < %zu needed",
                ctx->ws_bytes, need);
  return route_launch(ctx, logits, T_, E, k, topk_idx, gates, counts, offsets, row_of, src_tk,
                      reinterpret_cast<int32_t*>(ctx->ws));
}

moe_status moe_route_noalloc(moe_ctx* ctx, const float* logits, int T_, int E, int k,
                             int32_t* topk_idx, float* gates, int32_t* counts, int32_t* offsets,
                             int32_t* row_of, int32_t* src_tk) {
  moe_status st = route_validate(ctx, logits, T_, E, k, topk_idx, gates, counts, offsets, row_of, src_tk);
  if (st != MOE_OK) return st;
  const size_t nblk = (size_t)(T_ + kTokBlock - 1) / kTokBlock;
  if ((size_t)E * nblk > kScratchInts)
    return fail(ctx, MOE_ERR_UNSUPPORTED,
                "moe_route_noalloc: E * ceil(T/64) = %zu exceeds the %zu-entry scratch (T=%d E=%d)",
                (size_t)E * nblk, kScratchInts, T_, E);
  int32_t* bc = nullptr;
  st = scratch_address(ctx, &bc);
  if (st != MOE_OK) return st;
  return route_launch(ctx, logits, T_, E, k, topk_idx, gates, counts, offsets, row_of, src_tk, bc);
}

moe_status moe_route_bwd(moe_ctx* ctx, const float* gates, const float* dgates, int T_, int k,
                         float* dlogits_sel) {
  MOE_CHECK_CTX(ctx);
  MOE_REQUIRE(ctx, T_ >= 0 && k >= 1 && k <= 32, "moe_route_bwd: bad shape T=%d k=%d", T_, k);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, gates, T_ == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, dgates, T_ == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, dlogits_sel, T_ == 0);
  if (T_ == 0) return MOE_OK;
  moe_prof_scope ps(ctx, MOE_K_ROUTE_BWD);
  route_bwd_kernel<<<(T_ + 255) / 256, 256, 0, ctx->stream>>>(gates, dgates, T_, k, dlogits_sel,
                                                                nullptr, nullptr);
  return check_launch(ctx, "moe_route_bwd");
}

moe_status moe_route_bwd_rows(moe_ctx* ctx, const float* gates, const float* dgates,
                              const int32_t* row_of, int T_, int k, float* dlogits_sel,
                              float* dl_rows) {
  MOE_CHECK_CTX(ctx);
  MOE_REQUIRE(ctx, T_ >= 0 && k >= 1 && k <= 32, "moe_route_bwd_rows: bad shape T=%d k=%d", T_, k);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, gates, T_ == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, dgates, T_ == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, row_of, T_ == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, dlogits_sel, T_ == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, dl_rows, T_ == 0);
  MOE_REQUIRE_DISJOINT(ctx, "moe_route_bwd_rows", {dlogits_sel, (size_t)T_ * k * 4, "dlogits_sel"},
                       {dl_rows, (size_t)T_ * k * 4, "dl_rows"});
  if (T_ == 0) return MOE_OK;
  moe_prof_scope ps(ctx, MOE_K_ROUTE_BWD);
  route_bwd_kernel<<<(T_ + 255) / 256, 256, 0, ctx->stream>>>(gates, dgates, T_, k, dlogits_sel,
                                                                row_of, dl_rows);
  return check_launch(ctx, "moe_route_bwd_rows");
}

moe_status moe_router_wgrad(moe_ctx* ctx, const void* x, const float* dlogits_sel,
                            const int32_t* src_tk, const int32_t* offsets, int T_, int d, int E,
                            int k, moe_dtype dtype, void* dw_router) {
  MOE_CHECK_CTX(ctx);
  MOE_REQUIRE_DTYPE(ctx, dtype);
  MOE_REQUIRE(ctx, T_ >= 0 && d >= 8 && d % 8 == 0 && E >= 1 && E <= 1024 && k >= 1 && k <= E,
              "moe_router_wgrad: bad shape");
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, x, T_ == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, dlogits_sel, T_ == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, src_tk, T_ == 0);
  MOE_REQUIRE_PTR(ctx, offsets);
  MOE_REQUIRE_PTR(ctx, dw_router);
  const size_t need = router_wgrad_ws_bytes(T_, d, E, k);
  if (T_ > 0 && (ctx->ws == nullptr || ctx->ws_bytes < need))
    return fail(ctx, MOE_ERR_WORKSPACE, "moe_router_wgrad: workspace %zu bytes < %zu needed",
                ctx->ws_bytes, need);
  const int fc = dtype == MOE_BF16 ? 512 : 256;  // features per block (64 lanes x 16 bytes)
  float* part = reinterpret_cast<float*>(ctx->ws);
  int32_t* cstart = T_ > 0 ? reinterpret_cast<int32_t*>(
                                 reinterpret_cast<char*>(ctx->ws) +
                                 (((size_t)rw_chunk_bound(T_ * k, E) * d * sizeof(float) + 255) & ~(size_t)255))
                           : nullptr;
  const long long n2 = (long long)d * E;
  moe_prof_scope ps(ctx, MOE_K_ROUTER_WGRAD);
  if (T_ > 0) {
    dim3 grid((d + fc - 1) / fc, rw_chunk_bound(T_ * k, E));
    if (dtype == MOE_BF16)
      router_wgrad_part_kernel<bf16_t><<<grid, 256, 0, ctx->stream>>>(
          (const bf16_t*)x, dlogits_sel, src_tk, offsets, d, E, k, part, cstart);
    else
      router_wgrad_part_kernel<float><<<grid, 256, 0, ctx->stream>>>(
          (const float*)x, dlogits_sel, src_tk, offsets, d, E, k, part, cstart);
  }
  if (dtype == MOE_BF16)
    router_wgrad_sum_kernel<bf16_t><<<(unsigned)((n2 + 255) / 256), 256, 0, ctx->stream>>>(
        part, cstart, d, E, (bf16_t*)dw_router);
  else
    router_wgrad_sum_kernel<float><<<(unsigned)((n2 + 255) / 256), 256, 0, ctx->stream>>>(
        part, cstart, d, E, (float*)dw_router);
  return check_launch(ctx, "moe_router_wgrad");
}

}  // extern "C"
