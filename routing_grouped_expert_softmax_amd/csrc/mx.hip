// mx.hip — MXFP8 quantisation: E4M3 elements in 32-element blocks sharing an
// e8m0 (power-of-two) scale, for the expert GEMMs ([P1] 三, MXFP8).
//
// Scale rule (OCP MX): s = floor(log2(amax)) - 8, clamped to [-127, 127]
// (8 is the exponent of E4M3's largest normal 448 = 1.75 * 2^8); the scale
// byte is s + 127, so a zero block gets byte 0.  Elements are v / 2^s rounded
// to the nearest E4M3 value (ties to even), saturating at +-448, sign kept.
//
// Two layouts, both K-contiguous for the GEMM that consumes them:
//  * rowwise:  blocks along each row  -> codes [rows][cols], scales [rows][cols/32]
//  * columns:  blocks of 32 consecutive rows of one column, restarting at each
//    group of rows (an expert's tokens, or one expert's weight matrix), the
//    last block of a group zero-padded.  Output transposed:
//    codes [cols][Kpad], scales [cols][Kpad/32], where group g owns K
//    positions [P_g, P_g + roundup(n_g, 128)) and P is the exclusive scan of
//    the padded group sizes (128-padding keeps every 4-block scale word
//    aligned; padding blocks are zero codes with scale byte 0).
#include <hip/hip_runtime.h>

#include "common.h"
#include "mx.h"

using namespace moe;

namespace {

// Scale byte of a block from its largest magnitude: the float exponent field
// of amax minus 8, clamped to [0, 254] (0 also for amax == 0 or subnormal).
__device__ __forceinline__ int mx_scale_byte(float amax) {
  const int ef = (int)((__float_as_uint(amax) >> 23) & 0xff);
  const int c = ef - 8;
  return c < 0 ? 0 : (c > 254 ? 254 : c);
}

// E4M3 codes of four values already divided by the block scale, packed in
// element order: the hardware conversion (v_cvt_pk_fp8_f32, OCP E4M3, round
// to nearest even) of the values clamped to +-448, which is the saturating
// encoding of every value but NaN (the clamp turns a NaN into a bound).
// Checked on every bf16 bit pattern against a plain encoder that rounds each
// value to its binade's grid: equal for all non-NaN inputs, signed zeros and
// subnormals included.
__device__ __forceinline__ uint32_t e4m3x4_finite(float a, float b, float c, float d) {
  const float lo = -448.0f, hi = 448.0f;
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(a, lo, hi),
                                          __builtin_amdgcn_fmed3f(b, lo, hi), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(c, lo, hi),
                                      __builtin_amdgcn_fmed3f(d, lo, hi), w, true);
  return (uint32_t)w;
}

// The same with NaN kept: a NaN element becomes 0x7f.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  uint32_t r = e4m3x4_finite(a, b, c, d);
  if (a != a) r = (r & 0xffffff00u) | 0x0000007fu;
  if (b != b) r = (r & 0xffff00ffu) | 0x00007f00u;
  if (c != c) r = (r & 0xff00ffffu) | 0x007f0000u;
  if (d != d) r = (r & 0x00ffffffu) | 0x7f000000u;
  return r;
}

// Codes of one 32-element block f scaled by inv = 2^-s, as eight words.  A
// NaN is rare, so the block is encoded without the per-element NaN fix-ups
// and encoded again with them only when one of its elements is NaN (one
// unordered compare per pair of elements finds that).
__device__ __forceinline__ void e4m3_block(const float (&f)[32], float inv, uint32_t* out) {
  bool nan = false;
#pragma unroll
  for (int i = 0; i < 16; ++i) nan |= __builtin_isunordered(f[2 * i], f[2 * i + 1]);
#pragma unroll
  for (int q = 0; q < 8; ++q)
    out[q] = e4m3x4_finite(f[q * 4] * inv, f[q * 4 + 1] * inv, f[q * 4 + 2] * inv, f[q * 4 + 3] * inv);
  if (nan) {
#pragma unroll
    for (int q = 0; q < 8; ++q)
      out[q] = e4m3x4(f[q * 4] * inv, f[q * 4 + 1] * inv, f[q * 4 + 2] * inv, f[q * 4 + 3] * inv);
  }
}

// 2^-s as a float for a block scale exponent s in [-127, 127] (a normal
// number for every s the scale byte can give a bf16 block: s <= 119).
__device__ __forceinline__ float pow2_neg(int s) { return __uint_as_float((uint32_t)(127 - s) << 23); }

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Quantise one 32-element block held as four 16-byte bf16 chunks: the eight
// code words (four codes each, element order) and the scale byte.
__device__ __forceinline__ int quant_block(const uint4 (&v)[4], uint32_t (&out)[8]) {
  float f[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[i * 8 + 2 * j] = bf_lo(w[j]);
      f[i * 8 + 2 * j + 1] = bf_hi(w[j]);
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(f[i]));
  const int sb = mx_scale_byte(amax);
  const float inv = pow2_neg(sb - 127);
  e4m3_block(f, inv, out);
  return sb;
}

// One thread per 32-element block along a row.
__global__ void mx_rows_kernel(const uint4* __restrict__ src, long long nblocks, int bpr,
                               uint4* __restrict__ codes, uint8_t* __restrict__ scales) {
  const long long b = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  uint4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = src[b * 4 + i];
  uint32_t out[8];
  const int sb = quant_block(v, out);
  codes[b * 2] = make_uint4(out[0], out[1], out[2], out[3]);
  codes[b * 2 + 1] = make_uint4(out[4], out[5], out[6], out[7]);
  scales[b] = (uint8_t)sb;
  (void)bpr;
}

// Quantise-on-permute: thread b takes block b % bpr of token b / bpr, reads
// it once, quantises it once and writes the codes, the scale byte and
// (when xp is given) the bf16 block into each of the token's k expert rows.
__global__ void permute_mx_kernel(const uint4* __restrict__ x, const int32_t* __restrict__ row_of,
                                  long long nblocks, int bpr, int k, uint4* __restrict__ xp,
                                  uint4* __restrict__ codes, uint8_t* __restrict__ scales) {
  const long long b = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  const long long t = b / bpr;
  const int c = (int)(b - t * bpr);
  uint4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = x[b * 4 + i];
  uint32_t out[8];
  const int sb = quant_block(v, out);
  const uint4 c0 = make_uint4(out[0], out[1], out[2], out[3]);
  const uint4 c1 = make_uint4(out[4], out[5], out[6], out[7]);
  for (int j = 0; j < k; ++j) {
    const long long dst = (long long)row_of[t * k + j] * bpr + c;
    if (xp) {
#pragma unroll
      for (int i = 0; i < 4; ++i) xp[dst * 4 + i] = v[i];
    }
    codes[dst * 2] = c0;
    codes[dst * 2 + 1] = c1;
    scales[dst] = (uint8_t)sb;
  }
}

// Column blocks with groups.  Block (x = 128-column tile, y = 128-deep slice
// of the padded K space).  The slice's 128 x 128 bf16 source tile is staged in
// LDS with 16-byte row loads (eight in flight per thread; 32 KiB, so four
// blocks fit on a CU and one block's loads overlap another's quantisation);
// then two threads share each column, each quantising two 32-row blocks:
// half a 128-byte line of codes and two scale bytes.  Group g occupies padded
// K [P_g, P_g + roundup(n_g, 128)), so a slice lies in exactly one group; its
// rows past n_g are zeros (code 0, scale byte 0).  The slice's group comes
// from the padded group sizes: a closed form when every group has `urows`
// rows (offsets null), else a shuffle scan by wave 0.
// ROWS: the same read also yields the rowwise layout (rcodes [rows, cols],
// rscales [rows, cols/32], as mx_rows_kernel writes them).  A 32-column
// block of a row is the 16-byte chunks of four consecutive lanes in the
// staging loads, so its amax is two shuffles away; each lane encodes and
// stores its own eight codes.
constexpr int kColTile = 128;
template <bool ROWS>
__global__ void __launch_bounds__(256) mx_cols_kernel(
    const bf16_t* __restrict__ src, int rows, int cols, const int32_t* __restrict__ offsets,
    int urows, int G, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, int kpad_ld,
    uint8_t* __restrict__ rcodes, uint8_t* __restrict__ rscales) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[128 * kColTile];
  __shared__ int sh[4];
  const int tid = threadIdx.x;
  const int y = blockIdx.y;
  // The block's (group, 128-row slice): closed form for equal groups; else
  // wave 0 scans the per-group slice counts with shuffles (16 groups per
  // lane) and publishes the result through one barrier.
  int g, sl;
  if (offsets == nullptr) {
    const int pg = (urows + 127) / 128;  // slices per group
    if (pg == 0 || y >= G * pg) return;
    g = y / pg;
    sl = y - g * pg;
  } else {
    if (tid < 64) {
      const int lane = tid;
      const int per = (G + 63) / 64;  // <= 16 (G <= 1024)
      int cnt[16];
      int local = 0;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int gg = lane * per + q;
        cnt[q] = (q < per && gg < G) ? (offsets[gg + 1] - offsets[gg] + 127) / 128 : 0;
        local += cnt[q];
      }
      int incl = local;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off, 64);
        if (lane >= off) incl += v;
      }
      if (lane == 0) sh[0] = -1;
      int prun = incl - local;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        if (cnt[q] > 0 && y >= prun && y < prun + cnt[q]) {
          sh[0] = lane * per + q;
          sh[1] = y - prun;  // slice within the group
        }
        prun += cnt[q];
      }
    }
    __syncthreads();
    if (sh[0] < 0) return;
    g = sh[0];
    sl = sh[1];
  }
  const int gstart = offsets ? offsets[g] : g * urows;
  const int gend = offsets ? offsets[g + 1] : (g + 1) * urows;
  const int c0 = blockIdx.x * kColTile;
  const int r0 = gstart + sl * 128;
  const int nvalid = min(128, gend - r0);  // >= 1
  // stage: chunk i = (row i / 16, 8 columns (i % 16) * 8), zeros outside
  {
    uint4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = tid + 256 * j;
      const int row = i >> 4, col = c0 + (i & 15) * 8;
      v[j] = (row < nvalid && col < cols)
                 ? *reinterpret_cast<const uint4*>(src + (size_t)(r0 + row) * cols + col)
                 : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) reinterpret_cast<uint4*>(tile)[tid + 256 * j] = v[j];
    if (ROWS) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = tid + 256 * j;
        const int row = i >> 4, col = c0 + (i & 15) * 8;
        const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
        float f[8];
        float amax = 0.f;
        bool nan = false;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f[2 * q] = bf_lo(w[q]);
          f[2 * q + 1] = bf_hi(w[q]);
          amax = fmaxf(amax, fmaxf(fabsf(f[2 * q]), fabsf(f[2 * q + 1])));
          nan |= __builtin_isunordered(f[2 * q], f[2 * q + 1]);
        }
        // lanes 4m .. 4m+3 hold the block's four chunks (every lane takes part)
        amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
        const int sb = mx_scale_byte(amax);
        const float inv = pow2_neg(sb - 127);
        uint32_t c0w = e4m3x4_finite(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv);
        uint32_t c1w = e4m3x4_finite(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv);
        if (nan) {
          c0w = e4m3x4(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv);
          c1w = e4m3x4(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv);
        }
        if (row < nvalid && col < cols) {
          const size_t r = (size_t)(r0 + row);
          *reinterpret_cast<uint2*>(rcodes + r * cols + col) = make_uint2(c0w, c1w);
          if ((i & 3) == 0) rscales[r * (cols / 32) + col / 32] = (uint8_t)sb;
        }
      }
    }
  }
  __syncthreads();
  // thread -> (column cl, row half h): blocks 2h and 2h+1 of the column
  const int cl = tid & (kColTile - 1), h = tid >> 7;
  const int c = c0 + cl;
  uint32_t code_words[16];
  uint32_t sword = 0;
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    const int blk = 2 * h + bb;
    float f[32];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      f[i] = __uint_as_float(((uint32_t)tile[(blk * 32 + i) * kColTile + cl]) << 16);
      amax = fmaxf(amax, fabsf(f[i]));
    }
    const int sb = mx_scale_byte(amax);
    const float inv = pow2_neg(sb - 127);
    sword |= (uint32_t)sb << (8 * bb);
    e4m3_block(f, inv, code_words + bb * 8);
  }
  const size_t k = (size_t)y * 128;  // padded K position of the slice
  if (c < cols)
    *reinterpret_cast<uint16_t*>(scales + (size_t)c * (kpad_ld / 32) + k / 32 + 2 * h) = (uint16_t)sword;
  // codes go back through LDS (144-byte line pitch against bank conflicts) so
  // that each store instruction writes eight whole 128-byte lines
  constexpr int LP = 144;
  __syncthreads();  // every column has been read out of the tile
  unsigned char* lines = reinterpret_cast<unsigned char*>(tile);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<uint4*>(lines + cl * LP + 64 * h + 16 * i) =
        make_uint4(code_words[4 * i], code_words[4 * i + 1], code_words[4 * i + 2],
                   code_words[4 * i + 3]);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int piece = tid + 256 * j, line = piece >> 3, part = piece & 7;
    if (c0 + line < cols)
      *reinterpret_cast<uint4*>(codes + (size_t)(c0 + line) * kpad_ld + k + 16 * part) =
          *reinterpret_cast<const uint4*>(lines + line * LP + 16 * part);
  }
}

}  // namespace

using namespace moe_host;

// Upper bound of the padded K of a column-quantised operand.
long long mx_kpad_bound(int rows, int groups) { return (long long)rows + 127LL * groups + 127; }

hipError_t mx_quantize_rows(const void* src, int rows, int cols, uint8_t* codes, uint8_t* scales,
                            hipStream_t s) {
  const long long nb = (long long)rows * (cols / 32);
  if (nb == 0) return hipSuccess;
  mx_rows_kernel<<<(unsigned)((nb + 255) / 256), 256, 0, s>>>((const uint4*)src, nb, cols / 32,
                                                             (uint4*)codes, scales);
  return hipGetLastError();
}

hipError_t mx_quantize_cols(const void* src, int rows, int cols, const int32_t* offsets, int urows,
                            int groups, uint8_t* codes, uint8_t* scales, int kpad_ld,
                            hipStream_t s) {
  // bound on the padded slices: sum_g ceil(n_g / 128) <= rows / 128 + groups
  const int yb = rows / 128 + groups + 1;
  dim3 grid((cols + kColTile - 1) / kColTile, yb);
  mx_cols_kernel<false><<<grid, 256, 0, s>>>((const bf16_t*)src, rows, cols, offsets, urows, groups,
                                             codes, scales, kpad_ld, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t mx_quantize_both(const void* src, int rows, int cols, const int32_t* offsets, int urows,
                            int groups, uint8_t* codes, uint8_t* scales, int kpad_ld,
                            uint8_t* rcodes, uint8_t* rscales, hipStream_t s) {
  const int yb = rows / 128 + groups + 1;
  dim3 grid((cols + kColTile - 1) / kColTile, yb);
  mx_cols_kernel<true><<<grid, 256, 0, s>>>((const bf16_t*)src, rows, cols, offsets, urows, groups,
                                            codes, scales, kpad_ld, rcodes, rscales);
  return hipGetLastError();
}

extern "C" moe_status moe_permute_mx(moe_ctx* ctx, const void* x, const int32_t* row_of, int T_,
                                     int d, int k, void* xp, uint8_t* xp_codes, uint8_t* xp_scales) {
  MOE_CHECK_CTX(ctx);
  MOE_REQUIRE(ctx, T_ >= 0 && d >= 32 && d % 32 == 0 && k >= 1 && k <= 32 &&
                       (long long)T_ * k < (1LL << 31),
              "moe_permute_mx: bad shape T=%d d=%d k=%d (d %% 32 == 0)", T_, d, k);
  if (T_ == 0) return MOE_OK;
  MOE_REQUIRE_PTR(ctx, x);
  MOE_REQUIRE_PTR(ctx, row_of);
  MOE_REQUIRE_PTR(ctx, xp_codes);
  MOE_REQUIRE(ctx, xp_scales != nullptr, "moe_permute_mx: xp_scales is null");
  MOE_REQUIRE(ctx, xp == nullptr || aligned16(xp), "moe_permute_mx: xp not 16-byte aligned");
  {
    const size_t n = (size_t)T_ * k * d;
    MOE_REQUIRE_DISJOINT(ctx, "moe_permute_mx", {xp, n * 2, "xp"}, {xp_codes, n, "xp_codes"},
                         {xp_scales, n / 32, "xp_scales"});
  }
  const long long nb = (long long)T_ * (d / 32);
  moe_prof_scope ps(ctx, MOE_K_PERMUTE);
  permute_mx_kernel<<<(unsigned)((nb + 255) / 256), 256, 0, ctx->stream>>>(
      (const uint4*)x, row_of, nb, d / 32, k, (uint4*)xp, (uint4*)xp_codes, xp_scales);
  return check_launch(ctx, "moe_permute_mx");
}

extern "C" moe_status moe_mx_quantize(moe_ctx* ctx, const void* src_bf16, int rows, int cols,
                                      int axis, const int32_t* group_offsets, int groups,
                                      uint8_t* codes, uint8_t* scales_e8m0, int kpad_ld) {
  MOE_CHECK_CTX(ctx);
  MOE_REQUIRE(ctx, rows >= 0 && cols >= 32 && cols % 32 == 0, "moe_mx_quantize: bad shape");
  MOE_REQUIRE(ctx, axis == 0 || axis == 1, "moe_mx_quantize: axis must be 0 or 1");
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, src_bf16, rows == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, codes, rows == 0);
  MOE_REQUIRE(ctx, rows == 0 || scales_e8m0 != nullptr, "moe_mx_quantize: scales is null");
  if (rows == 0) return MOE_OK;
  if (axis == 0) {
    MOE_REQUIRE_DISJOINT(ctx, "moe_mx_quantize", {codes, (size_t)rows * cols, "codes"},
                         {scales_e8m0, (size_t)rows * cols / 32, "scales"});
  } else if (kpad_ld > 0) {
    MOE_REQUIRE_DISJOINT(ctx, "moe_mx_quantize", {codes, (size_t)cols * kpad_ld, "codes"},
                         {scales_e8m0, (size_t)cols * (kpad_ld / 32), "scales"});
  }
  moe_prof_scope ps(ctx, MOE_K_MX_QUANT);
  hipError_t e;
  if (axis == 0) {
    e = mx_quantize_rows(src_bf16, rows, cols, codes, scales_e8m0, ctx->stream);
  } else {
    MOE_REQUIRE(ctx, groups >= 1 && groups <= 1024, "moe_mx_quantize: 1 <= groups <= 1024");
    MOE_REQUIRE(ctx, group_offsets != nullptr || groups == 1,
                "moe_mx_quantize: group_offsets is null with groups > 1");
    MOE_REQUIRE(ctx, kpad_ld % 128 == 0 && kpad_ld >= mx_kpad_bound(rows, groups) - 127,
                "moe_mx_quantize: kpad_ld %d too small or not a multiple of 128", kpad_ld);
    e = mx_quantize_cols(src_bf16, rows, cols, group_offsets, group_offsets ? 0 : rows, groups,
                         codes, scales_e8m0, kpad_ld, ctx->stream);
  }
  if (e != hipSuccess) return fail(ctx, MOE_ERR_HIP, "moe_mx_quantize: %s", hipGetErrorString(e));
  return MOE_OK;
}

extern "C" moe_status moe_mx_quantize_both(moe_ctx* ctx, const void* src_bf16, int rows, int cols,
                                           const int32_t* group_offsets, int groups,
                                           uint8_t* codes_cols, uint8_t* scales_cols, int kpad_ld,
                                           uint8_t* codes_rows, uint8_t* scales_rows) {
  MOE_CHECK_CTX(ctx);
  MOE_REQUIRE(ctx, rows >= 0 && cols >= 32 && cols % 32 == 0, "moe_mx_quantize_both: bad shape");
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, src_bf16, rows == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, codes_cols, rows == 0);
  MOE_REQUIRE_PTR_OR_EMPTY(ctx, codes_rows, rows == 0);
  MOE_REQUIRE(ctx, rows == 0 || (scales_cols != nullptr && scales_rows != nullptr),
              "moe_mx_quantize_both: scales are null");
  if (rows == 0) return MOE_OK;
  MOE_REQUIRE(ctx, groups >= 1 && groups <= 1024, "moe_mx_quantize_both: 1 <= groups <= 1024");
  MOE_REQUIRE(ctx, group_offsets != nullptr || groups == 1,
              "moe_mx_quantize_both: group_offsets is null with groups > 1");
  MOE_REQUIRE(ctx, kpad_ld % 128 == 0 && kpad_ld >= mx_kpad_bound(rows, groups) - 127,
              "moe_mx_quantize_both: kpad_ld %d too small or not a multiple of 128", kpad_ld);
  MOE_REQUIRE_DISJOINT(ctx, "moe_mx_quantize_both", {codes_cols, (size_t)cols * kpad_ld, "codes_cols"},
                       {scales_cols, (size_t)cols * (kpad_ld / 32), "scales_cols"},
                       {codes_rows, (size_t)rows * cols, "codes_rows"},
                       {scales_rows, (size_t)rows * cols / 32, "scales_rows"});
  moe_prof_scope ps(ctx, MOE_K_MX_QUANT);
  const hipError_t e = mx_quantize_both(src_bf16, rows, cols, group_offsets, group_offsets ? 0 : rows,
                                        groups, codes_cols, scales_cols, kpad_ld, codes_rows,
                                        scales_rows, ctx->stream);
  if (e != hipSuccess) return fail(ctx, MOE_ERR_HIP, "moe_mx_quantize_both: %s", hipGetErrorString(e));
  return MOE_OK;
}
