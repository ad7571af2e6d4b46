// oracle.cpp — plain, slow CPU oracle of the dropless MoE feed-forward layer.
//
// TEST INFRASTRUCTURE ONLY: loaded by the test suite, the smoke check and the
// benchmark's CPU-baseline leg, never by the product path.  Plain loops, no
// BLAS, no intrinsics, no fast-math; OpenMP only over independent outer
// loops.  Every function follows the definition it cites (page keys in
// oracle.h).  It builds no expert buffers for the whole layer: each token is
// taken through its k experts one by one.
//
// Readings of the pages that are not fixed by them (taken here and listed
// with the design notes): selection on the float logits with the lower expert
// index first on ties (+0 and -0 tie); slot j is the j-th selected expert;
// gates are the softmax renormalised over the selected experts; rows inside an
// expert buffer are in ascending (t*k+j); the expert is SwiGLU without biases;
// the gate multiplies at the combine only; gradients of unselected logits are
// exactly zero.
#include "oracle.h"

#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

namespace {

template <class A>
inline A silu(A z) { return z / (A(1) + std::exp(-z)); }

template <class A>
inline A sigmoid(A z) { return A(1) / (A(1) + std::exp(-z)); }

// d silu(z) / dz = s(z) * (1 + z * (1 - s(z)))
template <class A>
inline A dsilu(A z) {
  A s = sigmoid(z);
  return s * (A(1) + z * (A(1) - s));
}

inline int expert_of_row(const int32_t* offsets, int E, int r) {
  // The expert whose segment [offsets[e], offsets[e+1]) holds row r.
  for (int e = 0; e < E; ++e)
    if (r >= offsets[e] && r < offsets[e + 1]) return e;
  return -1;
}

// ---------------------------------------------------------------- router
// Router logits: the router scores every token against every expert
// ([P2 1.1, 2.1]).  A linear router with no bias.
template <class A>
void router_logits(const float* x, const float* wr, int T, int d, int E, float* logits) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    for (int e = 0; e < E; ++e) {
      A s = 0;
      for (int i = 0; i < d; ++i) s += A(x[(size_t)t * d + i]) * A(wr[(size_t)i * E + e]);
      logits[(size_t)t * E + e] = float(s);
    }
  }
}

// True when expert a precedes expert b in the selection order of one token:
// larger logit first, lower index first when the logits are equal.
inline bool precedes(const float* l, int a, int b) {
  if (l[a] > l[b]) return true;
  if (l[a] < l[b]) return false;
  return a < b;
}

// Softmax over all E experts, top-k, renormalised gates ([P2 1.1, 2.1]), then
// the expert histogram, its exclusive scan and the stable permutation into
// expert-major rows (the "permutation index" of [P2 2.1]; routing metadata of
// [P1 二]).
template <class A>
void route(const float* logits, int T, int E, int k, int32_t* topk, double* gates, int32_t* counts,
           int32_t* offsets, int32_t* row_of, int32_t* src_tk) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    const float* l = logits + (size_t)t * E;
    // softmax probabilities
    A m = A(l[0]);
    for (int e = 1; e < E; ++e)
      if (A(l[e]) > m) m = A(l[e]);
    std::vector<A> p(E);
    A z = 0;
    for (int e = 0; e < E; ++e) {
      p[e] = std::exp(A(l[e]) - m);
      z += p[e];
    }
    for (int e = 0; e < E; ++e) p[e] /= z;
    // top-k by repeated selection of the first unselected expert in order
    std::vector<char> taken(E, 0);
    A psel = 0;
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || precedes(l, e, best)) best = e;
      }
      taken[best] = 1;
      topk[(size_t)t * k + j] = best;
      psel += p[best];
    }
    for (int j = 0; j < k; ++j) gates[(size_t)t * k + j] = double(p[topk[(size_t)t * k + j]] / psel);
  }
  // histogram and exclusive scan
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (size_t i = 0; i < (size_t)T * k; ++i) counts[topk[i]]++;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  // stable counting sort of the flat slot index t*k+j by expert
  std::vector<int32_t> cursor(offsets, offsets + E);
  for (size_t i = 0; i < (size_t)T * k; ++i) {
    int e = topk[i];
    int r = cursor[e]++;
    row_of[i] = r;
    src_tk[r] = (int32_t)i;
  }
}

// ---------------------------------------------------------------- expert
// One SwiGLU expert on one row: g = x*Wg, u = x*Wu, h = silu(g)*u, y = h*Wd.
template <class A>
void expert_row(const float* xr, int d, int F, const float* wg, const float* wu, const float* wd,
                A* g, A* u, A* h, A* y) {
  for (int f = 0; f < F; ++f) { g[f] = 0; u[f] = 0; }
  for (int i = 0; i < d; ++i) {
    A xi = A(xr[i]);
    const float* wgi = wg + (size_t)i * F;
    const float* wui = wu + (size_t)i * F;
    for (int f = 0; f < F; ++f) {
      g[f] += xi * A(wgi[f]);
      u[f] += xi * A(wui[f]);
    }
  }
  for (int f = 0; f < F; ++f) h[f] = silu(g[f]) * u[f];
  for (int c = 0; c < d; ++c) y[c] = 0;
  for (int f = 0; f < F; ++f) {
    A hf = h[f];
    const float* wdf = wd + (size_t)f * d;
    for (int c = 0; c < d; ++c) y[c] += hf * A(wdf[c]);
  }
}

// Backward of one expert on one row for upstream dy (d wide).
template <class A>
void expert_row_bwd(const float* xr, const float* dyr, int d, int F, const float* wg,
                    const float* wu, const float* wd, A* g, A* u, A* h, A* dg, A* du, A* dx) {
  std::vector<A> y(d), dh(F);
  expert_row<A>(xr, d, F, wg, wu, wd, g, u, h, y.data());
  for (int f = 0; f < F; ++f) {
    A s = 0;
    const float* wdf = wd + (size_t)f * d;
    for (int c = 0; c < d; ++c) s += A(dyr[c]) * A(wdf[c]);
    dh[f] = s;
  }
  for (int f = 0; f < F; ++f) {
    dg[f] = dh[f] * u[f] * dsilu(g[f]);
    du[f] = dh[f] * silu(g[f]);
  }
  for (int i = 0; i < d; ++i) {
    A s = 0;
    const float* wgi = wg + (size_t)i * F;
    const float* wui = wu + (size_t)i * F;
    for (int f = 0; f < F; ++f) s += dg[f] * A(wgi[f]) + du[f] * A(wui[f]);
    dx[i] = s;
  }
}

template <class A>
void expert_fwd(const float* xp, const int32_t* offsets, int E, int R, int d, int F, const float* wg,
                const float* wu, const float* wd, const int32_t* rows, int nrows, double* g,
                double* u, double* h, double* yp) {
  int n = rows ? nrows : R;
#pragma omp parallel
  {
    std::vector<A> gr(F), ur(F), hr(F), yr(d);
#pragma omp for schedule(dynamic, 4)
    for (int q = 0; q < n; ++q) {
      int r = rows ? rows[q] : q;
      int e = expert_of_row(offsets, E, r);
      const size_t wo = (size_t)e * d * F;
      expert_row<A>(xp + (size_t)r * d, d, F, wg + wo, wu + wo, wd + wo, gr.data(), ur.data(),
                    hr.data(), yr.data());
      // Outputs are indexed by position in the row list.
      for (int f = 0; f < F; ++f) {
        if (g) g[(size_t)q * F + f] = double(gr[f]);
        if (u) u[(size_t)q * F + f] = double(ur[f]);
        if (h) h[(size_t)q * F + f] = double(hr[f]);
      }
      if (yp)
        for (int c = 0; c < d; ++c) yp[(size_t)q * d + c] = double(yr[c]);
    }
  }
}

template <class A>
void expert_dgrad(const float* xp, const float* dyp, const int32_t* offsets, int E, int R, int d,
                  int F, const float* wg, const float* wu, const float* wd, const int32_t* rows,
                  int nrows, double* dg, double* du, double* dxp) {
  int n = rows ? nrows : R;
#pragma omp parallel
  {
    std::vector<A> gr(F), ur(F), hr(F), dgr(F), dur(F), dxr(d);
#pragma omp for schedule(dynamic, 4)
    for (int q = 0; q < n; ++q) {
      int r = rows ? rows[q] : q;
      int e = expert_of_row(offsets, E, r);
      const size_t wo = (size_t)e * d * F;
      expert_row_bwd<A>(xp + (size_t)r * d, dyp + (size_t)r * d, d, F, wg + wo, wu + wo, wd + wo,
                        gr.data(), ur.data(), hr.data(), dgr.data(), dur.data(), dxr.data());
      for (int f = 0; f < F; ++f) {
        if (dg) dg[(size_t)q * F + f] = double(dgr[f]);
        if (du) du[(size_t)q * F + f] = double(dur[f]);
      }
      if (dxp)
        for (int i = 0; i < d; ++i) dxp[(size_t)q * d + i] = double(dxr[i]);
    }
  }
}

// Weight gradients: every expert's rows are visited in ascending row order;
// experts are independent.
template <class A>
void expert_wgrad(const float* xp, const float* dyp, const int32_t* offsets, int E, int R, int d,
                  int F, const float* wg, const float* wu, const float* wd, double* dwg, double* dwu,
                  double* dwd) {
  (void)R;
  const size_t wsz = (size_t)d * F;
#pragma omp parallel for schedule(dynamic, 1)
  for (int e = 0; e < E; ++e) {
    std::vector<A> sg(wsz, A(0)), su(wsz, A(0)), sd(wsz, A(0));
    std::vector<A> g(F), u(F), h(F), dg(F), du(F), dx(d);
    const size_t wo = (size_t)e * wsz;
    for (int r = offsets[e]; r < offsets[e + 1]; ++r) {
      const float* xr = xp + (size_t)r * d;
      const float* dyr = dyp + (size_t)r * d;
      expert_row_bwd<A>(xr, dyr, d, F, wg + wo, wu + wo, wd + wo, g.data(), u.data(), h.data(),
                        dg.data(), du.data(), dx.data());
      for (int i = 0; i < d; ++i) {
        A xi = A(xr[i]);
        A* sgi = sg.data() + (size_t)i * F;
        A* sui = su.data() + (size_t)i * F;
        for (int f = 0; f < F; ++f) {
          sgi[f] += xi * dg[f];
          sui[f] += xi * du[f];
        }
      }
      for (int f = 0; f < F; ++f) {
        A hf = h[f];
        A* sdf = sd.data() + (size_t)f * d;
        for (int c = 0; c < d; ++c) sdf[c] += hf * A(dyr[c]);
      }
    }
    for (size_t q = 0; q < wsz; ++q) {
      dwg[wo + q] = double(sg[q]);
      dwu[wo + q] = double(su[q]);
      dwd[wo + q] = double(sd[q]);
    }
  }
}

// One weight-gradient element per entry, each summed over the expert's rows
// in row order, from the definitions of dg, du and h.
void expert_wgrad_elems(const float* xp, const float* dyp, const int32_t* offsets, int d, int F,
                        const float* wg, const float* wu, const float* wd, int which,
                        const int32_t* elem, int nelem, double* out) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int n = 0; n < nelem; ++n) {
    int e = elem[3 * n], a = elem[3 * n + 1], b = elem[3 * n + 2];
    const size_t wo = (size_t)e * d * F;
    const float* wge = wg + wo;
    const float* wue = wu + wo;
    const float* wde = wd + wo;
    // which 0/1: dW[e][i=a][f=b];  which 2: dWd[e][f=a][c=b]
    int f = (which == 2) ? a : b;
    double s = 0;
    for (int r = offsets[e]; r < offsets[e + 1]; ++r) {
      const float* xr = xp + (size_t)r * d;
      const float* dyr = dyp + (size_t)r * d;
      double g = 0, u = 0;
      for (int i = 0; i < d; ++i) {
        g += double(xr[i]) * double(wge[(size_t)i * F + f]);
        u += double(xr[i]) * double(wue[(size_t)i * F + f]);
      }
      if (which == 2) {
        s += silu(g) * u * double(dyr[b]);
        continue;
      }
      double dh = 0;
      for (int c = 0; c < d; ++c) dh += double(dyr[c]) * double(wde[(size_t)f * d + c]);
      double v = (which == 0) ? dh * u * dsilu(g) : dh * silu(g);
      s += double(xr[a]) * v;
    }
    out[n] = s;
  }
}

// ---------------------------------------------------------------- layer
template <class A>
void layer_fwd(const float* x, const int32_t* topk, const double* gates, int T, int d, int E, int k,
               int F, const float* wg, const float* wu, const float* wd, double* y, double* ytj) {
  (void)E;
#pragma omp parallel
  {
    std::vector<A> g(F), u(F), h(F), yo(d), acc(d);
#pragma omp for schedule(dynamic, 4)
    for (int t = 0; t < T; ++t) {
      for (int c = 0; c < d; ++c) acc[c] = 0;
      for (int j = 0; j < k; ++j) {
        int e = topk[(size_t)t * k + j];
        const size_t wo = (size_t)e * d * F;
        expert_row<A>(x + (size_t)t * d, d, F, wg + wo, wu + wo, wd + wo, g.data(), u.data(),
                      h.data(), yo.data());
        A gt = A(gates[(size_t)t * k + j]);
        for (int c = 0; c < d; ++c) acc[c] += gt * yo[c];
        if (ytj)
          for (int c = 0; c < d; ++c) ytj[((size_t)t * k + j) * d + c] = double(yo[c]);
      }
      for (int c = 0; c < d; ++c) y[(size_t)t * d + c] = double(acc[c]);
    }
  }
}

// Whole-layer backward in fp64.  Token loop for everything per token; the
// weight gradients are then accumulated per expert in ascending token order.
void layer_bwd(const float* x, const float* wr, const int32_t* topk, const double* gates,
               const float* dy, int T, int d, int E, int k, int F, const float* wg, const float* wu,
               const float* wd, double* dgates, double* dlogits_sel, double* dx, double* dwg,
               double* dwu, double* dwd, double* dwr) {
  const size_t wsz = (size_t)d * F;
  // Per (t,j): dg, du, h and dY kept for the weight gradients.
  std::vector<double> DG((size_t)T * k * F), DU((size_t)T * k * F), H((size_t)T * k * F);
#pragma omp parallel
  {
    std::vector<double> g(F), u(F), h(F), yo(d), dh(F), dgv(F), duv(F);
#pragma omp for schedule(dynamic, 4)
    for (int t = 0; t < T; ++t) {
      const float* xt = x + (size_t)t * d;
      const float* dyt = dy + (size_t)t * d;
      double* dxt = dx + (size_t)t * d;
      for (int i = 0; i < d; ++i) dxt[i] = 0;
      for (int j = 0; j < k; ++j) {
        const size_t tj = (size_t)t * k + j;
        int e = topk[tj];
        const size_t wo = (size_t)e * wsz;
        expert_row<double>(xt, d, F, wg + wo, wu + wo, wd + wo, g.data(), u.data(), h.data(),
                           yo.data());
        // gate gradient and the expert's upstream dY = gate * dy
        double dgt = 0;
        for (int c = 0; c < d; ++c) dgt += double(dyt[c]) * yo[c];
        dgates[tj] = dgt;
        const double gt = gates[tj];
        for (int f = 0; f < F; ++f) {
          double s = 0;
          const float* wdf = wd + wo + (size_t)f * d;
          for (int c = 0; c < d; ++c) s += gt * double(dyt[c]) * double(wdf[c]);
          dh[f] = s;
        }
        for (int f = 0; f < F; ++f) {
          dgv[f] = dh[f] * u[f] * dsilu(g[f]);
          duv[f] = dh[f] * silu(g[f]);
          DG[tj * F + f] = dgv[f];
          DU[tj * F + f] = duv[f];
          H[tj * F + f] = h[f];
        }
        for (int i = 0; i < d; ++i) {
          double s = 0;
          const float* wgi = wg + wo + (size_t)i * F;
          const float* wui = wu + wo + (size_t)i * F;
          for (int f = 0; f < F; ++f) s += dgv[f] * double(wgi[f]) + duv[f] * double(wui[f]);
          dxt[i] += s;
        }
      }
      // renormalised-softmax backward onto the selected logits
      double gd = 0;
      for (int j = 0; j < k; ++j) gd += gates[(size_t)t * k + j] * dgates[(size_t)t * k + j];
      for (int j = 0; j < k; ++j) {
        const size_t tj = (size_t)t * k + j;
        dlogits_sel[tj] = gates[tj] * (dgates[tj] - gd);
        const int e = topk[tj];
        for (int i = 0; i < d; ++i) dxt[i] += dlogits_sel[tj] * double(wr[(size_t)i * E + e]);
      }
    }
  }
  // weight gradients, one expert per iteration, tokens ascending
#pragma omp parallel for schedule(dynamic, 1)
  for (int e = 0; e < E; ++e) {
    double* sg = dwg + (size_t)e * wsz;
    double* su = dwu + (size_t)e * wsz;
    double* sd = dwd + (size_t)e * wsz;
    for (size_t q = 0; q < wsz; ++q) { sg[q] = 0; su[q] = 0; sd[q] = 0; }
    for (int i = 0; i < d; ++i) dwr[(size_t)i * E + e] = 0;
    for (int t = 0; t < T; ++t) {
      for (int j = 0; j < k; ++j) {
        const size_t tj = (size_t)t * k + j;
        if (topk[tj] != e) continue;
        const float* xt = x + (size_t)t * d;
        const float* dyt = dy + (size_t)t * d;
        const double gt = gates[tj];
        for (int i = 0; i < d; ++i) {
          double xi = double(xt[i]);
          for (int f = 0; f < F; ++f) {
            sg[(size_t)i * F + f] += xi * DG[tj * F + f];
            su[(size_t)i * F + f] += xi * DU[tj * F + f];
          }
          dwr[(size_t)i * E + e] += dlogits_sel[tj] * xi;
        }
        for (int f = 0; f < F; ++f)
          for (int c = 0; c < d; ++c) sd[(size_t)f * d + c] += H[tj * F + f] * gt * double(dyt[c]);
      }
    }
  }
}

// ---------------------------------------------------------------- MXFP8
// E4M3 "FN": 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent field 15
// with mantissa 7 is NaN, so the largest finite magnitude is 1.75 * 2^8 = 448;
// no infinities; subnormals are m * 2^-9.  Encoding is round-to-nearest-even
// on the float bit pattern, saturating to 448.
uint8_t e4m3_encode(float v) {
  uint32_t b;
  std::memcpy(&b, &v, 4);
  const uint8_t sign = (uint8_t)((b >> 31) << 7);
  const uint32_t mag = b & 0x7fffffffu;
  if (mag > 0x7f800000u) return 0x7f;  // NaN
  // Saturate: everything at or above 448 (0x43e00000), including +-inf,
  // maps to the largest finite code.
  if (mag >= 0x43e00000u) return (uint8_t)(sign | 0x7e);
  const int fexp = (int)(mag >> 23) - 127;  // unbiased float exponent
  if (fexp < -6) {
    // Subnormal E4M3 target: value = m * 2^-9 with m in 0..7 (m == 8 is the
    // smallest normal).  m = RNE(|v| * 2^9).  Work on the significand so the
    // rounding is exact: |v| = sig * 2^(fexp - 23), sig has the implicit bit.
    if (mag < 0x00800000u) return sign;  // float subnormal or zero: far below 2^-10
    uint32_t sig = (mag & 0x7fffffu) | 0x800000u;
    int shift = 23 - (fexp + 9);  // bits to drop so that units are 2^-9
    if (shift > 24) return sign;   // below half of 2^-9
    uint32_t q = sig >> shift;
    uint32_t rem = sig & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u))) q++;
    // q == 8 lands exactly on the smallest normal, whose code is 0x08.
    return (uint8_t)(sign | q);
  }
  // Normal range: keep 3 mantissa bits with RNE on the dropped 20 bits.
  uint32_t mant = mag & 0x7fffffu;
  uint32_t keep = mant >> 20;
  uint32_t rem = mant & 0xfffffu;
  int e = fexp + 7;  // biased E4M3 exponent, 1..15
  if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) {
    keep++;
    if (keep == 8) {
      keep = 0;
      e++;
    }
  }
  uint32_t code = ((uint32_t)e << 3) | keep;
  if (code > 0x7e) code = 0x7e;  // values rounding past 448 saturate
  return (uint8_t)(sign | code);
}

float e4m3_decode(uint8_t c) {
  const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return std::nanf("");
  float v = (e == 0) ? std::ldexp((float)m, -9) : std::ldexp(1.0f + m / 8.0f, e - 7);
  return s ? -v : v;
}

// Shared block scale: 2^s with s = floor(log2 amax) - 8, clamped to the e8m0
// range [-127, 127]; a zero block gets code 0.
uint8_t mx_scale_code(float amax) {
  if (!(amax > 0.0f)) return 0;
  int ex;
  std::frexp(amax, &ex);  // amax = f * 2^ex with f in [0.5, 1): floor(log2) = ex - 1
  int s = (ex - 1) - 8;
  if (s < -127) s = -127;
  if (s > 127) s = 127;
  return (uint8_t)(s + 127);
}

// Element code: the value divided by the block scale, encoded as E4M3.
uint8_t mx_encode_elem(float v, uint8_t scale) {
  const int s = (int)scale - 127;
  return e4m3_encode(std::ldexp(v, -s));
}

}  // namespace

extern "C" {

void oracle_router_logits_f64(const float* x, const float* wr, int T, int d, int E, float* l) {
  router_logits<double>(x, wr, T, d, E, l);
}
void oracle_router_logits_f32(const float* x, const float* wr, int T, int d, int E, float* l) {
  router_logits<float>(x, wr, T, d, E, l);
}
void oracle_route_f64(const float* l, int T, int E, int k, int32_t* ti, double* g, int32_t* c,
                      int32_t* o, int32_t* ro, int32_t* st) {
  route<double>(l, T, E, k, ti, g, c, o, ro, st);
}
void oracle_route_f32(const float* l, int T, int E, int k, int32_t* ti, double* g, int32_t* c,
                      int32_t* o, int32_t* ro, int32_t* st) {
  route<float>(l, T, E, k, ti, g, c, o, ro, st);
}
void oracle_expert_fwd_f64(const float* xp, const int32_t* off, int E, int R, int d, int F,
                           const float* wg, const float* wu, const float* wd, const int32_t* rows,
                           int nrows, double* g, double* u, double* h, double* yp) {
  expert_fwd<double>(xp, off, E, R, d, F, wg, wu, wd, rows, nrows, g, u, h, yp);
}
void oracle_expert_fwd_f32(const float* xp, const int32_t* off, int E, int R, int d, int F,
                           const float* wg, const float* wu, const float* wd, const int32_t* rows,
                           int nrows, double* g, double* u, double* h, double* yp) {
  expert_fwd<float>(xp, off, E, R, d, F, wg, wu, wd, rows, nrows, g, u, h, yp);
}
void oracle_expert_dgrad_f64(const float* xp, const float* dyp, const int32_t* off, int E, int R,
                             int d, int F, const float* wg, const float* wu, const float* wd,
                             const int32_t* rows, int nrows, double* dg, double* du, double* dxp) {
  expert_dgrad<double>(xp, dyp, off, E, R, d, F, wg, wu, wd, rows, nrows, dg, du, dxp);
}
void oracle_expert_dgrad_f32(const float* xp, const float* dyp, const int32_t* off, int E, int R,
                             int d, int F, const float* wg, const float* wu, const float* wd,
                             const int32_t* rows, int nrows, double* dg, double* du, double* dxp) {
  expert_dgrad<float>(xp, dyp, off, E, R, d, F, wg, wu, wd, rows, nrows, dg, du, dxp);
}
void oracle_expert_wgrad_f64(const float* xp, const float* dyp, const int32_t* off, int E, int R,
                             int d, int F, const float* wg, const float* wu, const float* wd,
                             double* dwg, double* dwu, double* dwd) {
  expert_wgrad<double>(xp, dyp, off, E, R, d, F, wg, wu, wd, dwg, dwu, dwd);
}
void oracle_expert_wgrad_f32(const float* xp, const float* dyp, const int32_t* off, int E, int R,
                             int d, int F, const float* wg, const float* wu, const float* wd,
                             double* dwg, double* dwu, double* dwd) {
  expert_wgrad<float>(xp, dyp, off, E, R, d, F, wg, wu, wd, dwg, dwu, dwd);
}
void oracle_expert_wgrad_elems_f64(const float* xp, const float* dyp, const int32_t* off, int E,
                                   int R, int d, int F, const float* wg, const float* wu,
                                   const float* wd, int which, const int32_t* elem, int nelem,
                                   double* out) {
  (void)E;
  (void)R;
  expert_wgrad_elems(xp, dyp, off, d, F, wg, wu, wd, which, elem, nelem, out);
}
void oracle_layer_fwd_f64(const float* x, const int32_t* topk, const double* gates, int T, int d,
                          int E, int k, int F, const float* wg, const float* wu, const float* wd,
                          double* y, double* ytj) {
  layer_fwd<double>(x, topk, gates, T, d, E, k, F, wg, wu, wd, y, ytj);
}
void oracle_layer_fwd_f32(const float* x, const int32_t* topk, const double* gates, int T, int d,
                          int E, int k, int F, const float* wg, const float* wu, const float* wd,
                          double* y, double* ytj) {
  layer_fwd<float>(x, topk, gates, T, d, E, k, F, wg, wu, wd, y, ytj);
}
void oracle_layer_bwd_f64(const float* x, const float* wr, const int32_t* topk, const double* gates,
                          const float* dy, int T, int d, int E, int k, int F, const float* wg,
                          const float* wu, const float* wd, double* dgates, double* dlogits_sel,
                          double* dx, double* dwg, double* dwu, double* dwd, double* dwr) {
  layer_bwd(x, wr, topk, gates, dy, T, d, E, k, F, wg, wu, wd, dgates, dlogits_sel, dx, dwg, dwu,
            dwd, dwr);
}

uint8_t oracle_e4m3_encode(float v) { return e4m3_encode(v); }
float oracle_e4m3_decode(uint8_t c) { return e4m3_decode(c); }
uint8_t oracle_mx_scale_code(float amax) { return mx_scale_code(amax); }

void oracle_mx_quantize(const float* src, int rows, int cols, int axis, const int32_t* offsets,
                        int groups, uint8_t* codes, uint8_t* scales) {
  if (axis == 0) {
    const int nb = cols / 32;
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; ++r) {
      for (int b = 0; b < nb; ++b) {
        const float* v = src + (size_t)r * cols + (size_t)b * 32;
        float amax = 0;
        for (int i = 0; i < 32; ++i) amax = std::fmax(amax, std::fabs(v[i]));
        uint8_t s = mx_scale_code(amax);
        scales[(size_t)r * nb + b] = s;
        for (int i = 0; i < 32; ++i)
          codes[(size_t)r * cols + (size_t)b * 32 + i] = mx_encode_elem(v[i], s);
      }
    }
    return;
  }
  // axis 1: blocks of 32 consecutive rows of one column inside each group;
  // padding rows past the group's end count as zeros.
  int ng = offsets ? groups : 1;
  std::vector<int> blk0(ng + 1, 0);
  for (int g = 0; g < ng; ++g) {
    int lo = offsets ? offsets[g] : 0, hi = offsets ? offsets[g + 1] : rows;
    blk0[g + 1] = blk0[g] + (hi - lo + 31) / 32;
  }
  for (int g = 0; g < ng; ++g) {
    int lo = offsets ? offsets[g] : 0, hi = offsets ? offsets[g + 1] : rows;
#pragma omp parallel for schedule(static)
    for (int c = 0; c < cols; ++c) {
      for (int b = 0; b < blk0[g + 1] - blk0[g]; ++b) {
        int r0 = lo + 32 * b, r1 = r0 + 32 < hi ? r0 + 32 : hi;
        float amax = 0;
        for (int r = r0; r < r1; ++r) amax = std::fmax(amax, std::fabs(src[(size_t)r * cols + c]));
        uint8_t s = mx_scale_code(amax);
        scales[(size_t)(blk0[g] + b) * cols + c] = s;
        for (int r = r0; r < r1; ++r)
          codes[(size_t)r * cols + c] = mx_encode_elem(src[(size_t)r * cols + c], s);
      }
    }
  }
}

}  // extern "C"
