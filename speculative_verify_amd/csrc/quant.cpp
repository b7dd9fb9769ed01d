// Host-side offline quantizers (declared in svq.h).
//
//   quantize_int4_frozen  the report's packing step (sec. 2.1): weights updated
//                         under frozen symmetric group scales go back onto the
//                         INT4 grid, each to its nearest grid point.
//   fit_binary_planes     the ShiftAddQwen README's binary-coding fit
//                         ("Output-aware fit"): greedy initialisation, then
//                         alternating least squares with exhaustive code choice,
//                         per (row, group), on the plain weight error.
//   snap_sa_scales        the README's sa* scale storage ("Format", "Scale
//                         distillation"): plane scales snapped onto u8 codes
//                         times one fp16 d per 256-weight super-block.
//
// All arithmetic is fp64 and every integer decision (a code, a sign vector)
// is taken in fp64, so the results do not depend on the thread count.
#include <cmath>
#include <cstdint>
#include <cstring>

#include "svq.h"
#include "svq_internal.h"

namespace {

inline double bf16_value(uint16_t h) {
  const uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

inline double f16_value(uint16_t h) {
  _Float16 v;
  std::memcpy(&v, &h, 2);
  return (double)v;
}

// IEEE binary16 bits of v, correctly rounded (nearest, ties to even).
inline uint16_t f16_bits(double v) {
  const _Float16 h = (_Float16)v;
  uint16_t b;
  std::memcpy(&b, &h, 2);
  return b;
}

// Nearest integer, ties to even (the default rounding mode of the host).
inline double round_even(double v) { return std::nearbyint(v); }

bool valid_group(int32_t G) { return G == 64 || G == 128 || G == 256; }

// One (row, group) of the plane fit.  w: G weights; b: P x G signs; a: P scales.
class PlaneFit {
 public:
  PlaneFit(const double* w, int G, int P) : w_(w), G_(G), P_(P) {}

  // Greedy start: each plane takes the signs of the residual (+1 at zero)
  // and the mean absolute residual as its scale, then leaves its part out.
  void greedy(int8_t* b, double* a) const {
    double r[256];
    for (int k = 0; k < G_; ++k) r[k] = w_[k];
    for (int p = 0; p < P_; ++p) {
      double sum_abs = 0.0;
      int8_t* bp = b + p * G_;
      for (int k = 0; k < G_; ++k) {
        bp[k] = r[k] < 0.0 ? -1 : 1;
        sum_abs += std::fabs(r[k]);
      }
      a[p] = sum_abs / G_;
      for (int k = 0; k < G_; ++k) r[k] -= a[p] * bp[k];
    }
  }

  // Every weight takes the sign vector whose value sum_p a_p b_p (planes
  // added in order) is nearest; the lowest candidate index wins a tie, where
  // bit p of the index set means b_p = -1.
  void choose_codes(const double* a, int8_t* b) const {
    const int nc = 1 << P_;
    double val[64];
    for (int c = 0; c < nc; ++c) {
      double v = 0.0;
      for (int p = 0; p < P_; ++p) v += (c >> p & 1) ? -a[p] : a[p];
      val[c] = v;
    }
    for (int k = 0; k < G_; ++k) {
      int best = 0;
      double best_d = std::fabs(w_[k] - val[0]);
      for (int c = 1; c < nc; ++c) {
        const double d = std::fabs(w_[k] - val[c]);
        if (d < best_d) {
          best_d = d;
          best = c;
        }
      }
      for (int p = 0; p < P_; ++p) b[p * G_ + k] = (best >> p & 1) ? -1 : 1;
    }
  }

  // Least-squares scales for the signs b: the normal equations
  // (B B^T) a = B w solved by a Cholesky factorisation.  A singular system
  // (one plane a combination of the others over this group) keeps a.
  void refit_scales(const int8_t* b, double* a) const {
    double gram[6][6], rhs[6], chol[6][6];
    for (int p = 0; p < P_; ++p) {
      const int8_t* bp = b + p * G_;
      double acc = 0.0;
      for (int k = 0; k < G_; ++k) acc += bp[k] * w_[k];
      rhs[p] = acc;
      for (int q = 0; q < P_; ++q) {
        const int8_t* bq = b + q * G_;
        int dot = 0;
        for (int k = 0; k < G_; ++k) dot += bp[k] * bq[k];
        gram[p][q] = dot;
      }
    }
    for (int i = 0; i < P_; ++i) {
      for (int j = 0; j < i; ++j) {
        double acc = gram[i][j];
        for (int t = 0; t < j; ++t) acc -= chol[i][t] * chol[j][t];
        chol[i][j] = acc / chol[j][j];
      }
      double acc = gram[i][i];
      for (int t = 0; t < i; ++t) acc -= chol[i][t] * chol[i][t];
      if (acc <= 1e-9 * G_) return;
      chol[i][i] = std::sqrt(acc);
    }
    double fwd[6];
    for (int i = 0; i < P_; ++i) {
      double acc = rhs[i];
      for (int t = 0; t < i; ++t) acc -= chol[i][t] * fwd[t];
      fwd[i] = acc / chol[i][i];
    }
    for (int i = P_ - 1; i >= 0; --i) {
      double acc = fwd[i];
      for (int t = i + 1; t < P_; ++t) acc -= chol[t][i] * a[t];
      a[i] = acc / chol[i][i];
    }
  }

 private:
  const double* w_;
  int G_, P_;
};

}  // namespace

extern "C" {

int quantize_int4_frozen(const uint16_t* w_bf16, const uint16_t* scales_bf16, int64_t N, int64_t K, int32_t G,
                         int8_t* codes) {
  svq::clear_error();
  if (!w_bf16 || !scales_bf16 || !codes) return svq::fail(SVQ_ERR_NULL, "quantize_int4_frozen: NULL pointer");
  if (N < 1 || !valid_group(G) || K < G || K % G)
    return svq::fail(SVQ_ERR_SHAPE, "quantize_int4_frozen: need N >= 1, G in {64, 128, 256}, K a multiple of G");
  const int64_t ng = K / G;
  svq::parallel_for(N, [&](int64_t lo, int64_t hi) {
    for (int64_t n = lo; n < hi; ++n)
      for (int64_t g = 0; g < ng; ++g) {
        const double s = bf16_value(scales_bf16[n * ng + g]);
        for (int64_t k = g * G; k < (g + 1) * G; ++k) {
          double c = 0.0;
          if (s != 0.0) c = std::fmin(7.0, std::fmax(-8.0, round_even(bf16_value(w_bf16[n * K + k]) / s)));
          codes[n * K + k] = (int8_t)c;
        }
      }
  });
  return SVQ_OK;
}

int fit_binary_planes(const uint16_t* w_bf16, int64_t N, int64_t K, int32_t G, int32_t P, int32_t iters,
                      int8_t* signs, uint16_t* alpha_f16) {
  svq::clear_error();
  if (!w_bf16 || !signs || !alpha_f16) return svq::fail(SVQ_ERR_NULL, "fit_binary_planes: NULL pointer");
  if (N < 1 || !valid_group(G) || K < G || K % G)
    return svq::fail(SVQ_ERR_SHAPE, "fit_binary_planes: need N >= 1, G in {64, 128, 256}, K a multiple of G");
  if (P < 1 || P > SVQ_MAX_P) return svq::fail(SVQ_ERR_SHAPE, "fit_binary_planes: P=%d must be in 1..6", P);
  if (iters < 0) return svq::fail(SVQ_ERR_SHAPE, "fit_binary_planes: iters=%d must be >= 0", iters);
  const int64_t ng = K / G;
  svq::parallel_for(N, [&](int64_t lo, int64_t hi) {
    double w[256], a[6];
    int8_t b[6 * 256], prev[6 * 256];
    for (int64_t n = lo; n < hi; ++n)
      for (int64_t g = 0; g < ng; ++g) {
        for (int k = 0; k < G; ++k) w[k] = bf16_value(w_bf16[n * K + g * G + k]);
        const PlaneFit fit(w, G, P);
        fit.greedy(b, a);
        for (int it = 0; it < iters; ++it) {
          std::memcpy(prev, b, (size_t)P * G);
          fit.choose_codes(a, b);
          // Unchanged signs give the same least-squares scales: a fixed point.
          if (it > 0 && std::memcmp(prev, b, (size_t)P * G) == 0) break;
          fit.refit_scales(b, a);
        }
        for (int p = 0; p < P; ++p) {
          const bool flip = a[p] < 0.0;
          alpha_f16[((int64_t)p * N + n) * ng + g] = f16_bits(flip ? -a[p] : a[p]);
          int8_t* out = signs + ((int64_t)p * N + n) * K + g * G;
          for (int k = 0; k < G; ++k) out[k] = (int8_t)(flip ? -b[p * G + k] : b[p * G + k]);
        }
      }
  });
  return SVQ_OK;
}

int snap_sa_scales(const uint16_t* alpha_f16, int64_t N, int64_t K, int32_t G, int32_t P, uint8_t* codes,
                   uint16_t* d_f16) {
  svq::clear_error();
  if (!alpha_f16 || !codes || !d_f16) return svq::fail(SVQ_ERR_NULL, "snap_sa_scales: NULL pointer");
  if (N < 1 || !valid_group(G) || K < 256 || K % 256)
    return svq::fail(SVQ_ERR_SHAPE, "snap_sa_scales: need N >= 1, G in {64, 128, 256}, K a multiple of 256");
  if (P < 1 || P > SVQ_MAX_P) return svq::fail(SVQ_ERR_SHAPE, "snap_sa_scales: P=%d must be in 1..6", P);
  const int64_t ng = K / G, ns = K / 256, per_sb = 256 / G;
  for (int64_t i = 0; i < (int64_t)P * N * ng; ++i)
    if (f16_value(alpha_f16[i]) < 0.0 || std::isnan(f16_value(alpha_f16[i])))
      return svq::fail(SVQ_ERR_RANGE, "snap_sa_scales: alpha at (p=%lld, n=%lld, g=%lld) is negative or NaN",
                       (long long)(i / (N * ng)), (long long)(i / ng % N), (long long)(i % ng));
  svq::parallel_for(N, [&](int64_t lo, int64_t hi) {
    for (int64_t n = lo; n < hi; ++n)
      for (int64_t j = 0; j < ns; ++j) {
        double top = 0.0;
        for (int p = 0; p < P; ++p)
          for (int64_t g = j * per_sb; g < (j + 1) * per_sb; ++g)
            top = std::fmax(top, f16_value(alpha_f16[((int64_t)p * N + n) * ng + g]));
        const uint16_t db = f16_bits(top / 255.0);
        const double d = f16_value(db);
        d_f16[n * ns + j] = db;
        for (int p = 0; p < P; ++p)
          for (int64_t g = j * per_sb; g < (j + 1) * per_sb; ++g) {
            const int64_t e = ((int64_t)p * N + n) * ng + g;
            codes[e] = (uint8_t)(d > 0.0 ? std::fmin(255.0, round_even(f16_value(alpha_f16[e]) / d)) : 0.0);
          }
      }
  });
  return SVQ_OK;
}

}  // extern "C"
