// Host side of libtq: the C ABI, argument validation, the float64 Lloyd-Max solver, the
// float64 Householder QR that turns a Gaussian draw into a Haar rotation, and the upload of
// the rotation's MFMA operand tiles.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cfloat>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <set>
#include <string>
#include <utility>
#include <vector>

#include "tq_internal.h"

namespace tq {

static thread_local std::string g_error;

void set_error(const std::string& msg) { g_error = msg; }

static int fail(int status, const std::string& msg) {
  set_error(msg);
  return status;
}

// ------------------------------------------------------------------------------------
// Gauss-Legendre rule on [-1, 1]: nodes are the roots of P_n, found by Newton's method
// from the Chebyshev-like first guess cos(pi (i + 3/4) / (n + 1/2)); weights
// 2 / ((1 - x^2) P_n'(x)^2).
struct GaussLegendre {
  std::vector<double> x, w;
  explicit GaussLegendre(int n) : x(n), w(n) {
    for (int i = 0; i < (n + 1) / 2; ++i) {
      double z = std::cos(M_PI * (i + 0.75) / (n + 0.5));
      double dp = 0.0;
      for (int it = 0; it < 100; ++it) {
        double p0 = 1.0, p1 = z;
        for (int k = 2; k <= n; ++k) {
          double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
          p0 = p1;
          p1 = p2;
        }
        dp = n * (z * p1 - p0) / (z * z - 1.0);
        double dz = p1 / dp;
        z -= dz;
        if (std::fabs(dz) < 1e-16) break;
      }
      {  // final derivative at the converged root
        double p0 = 1.0, p1 = z;
        for (int k = 2; k <= n; ++k) {
          double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
          p0 = p1;
          p1 = p2;
        }
        dp = n * (z * p1 - p0) / (z * z - 1.0);
      }
      x[i] = -z;
      x[n - 1 - i] = z;
      w[i] = w[n - 1 - i] = 2.0 / ((1.0 - z * z) * dp * dp);
    }
  }
};

// Density of one coordinate of a uniform unit vector in R^d:
// f(x) = C_d (1 - x^2)^((d-3)/2), C_d = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)).
struct SphereDensity {
  double log_c, m, sigma;
  explicit SphereDensity(int d)
      : log_c(std::lgamma(d / 2.0) - 0.5 * std::log(M_PI) - std::lgamma((d - 1) / 2.0)),
        m((d - 3) / 2.0),
        sigma(1.0 / std::sqrt((double)d)) {}
  double pdf(double x) const {
    if (std::fabs(x) >= 1.0) return 0.0;
    return std::exp(log_c + m * std::log1p(-x * x));
  }
};

// Integrals of x^p f(x) (p = 0, 1) and of (x - c)^2 f(x) over [a, b] by composite
// Gauss-Legendre (panels x nodes). Beyond 40 sigma the density is below e^-800 of its peak,
// so the range is clipped there.
struct CellIntegrator {
  const SphereDensity& f;
  GaussLegendre gl;
  int panels;
  CellIntegrator(const SphereDensity& f_, int nodes, int panels_) : f(f_), gl(nodes), panels(panels_) {}
  void integrate(double a, double b, double c, double* mass, double* first, double* sqerr) const {
    double lim = std::min(1.0, 40.0 * f.sigma);
    a = std::max(a, -lim);
    b = std::min(b, lim);
    double s0 = 0, s1 = 0, s2 = 0;
    if (b > a) {
      double h = (b - a) / panels;
      for (int p = 0; p < panels; ++p) {
        double lo = a + p * h, half = 0.5 * h, mid = lo + half;
        for (size_t i = 0; i < gl.x.size(); ++i) {
          double x = mid + half * gl.x[i];
          double wf = half * gl.w[i] * f.pdf(x);
          s0 += wf;
          s1 += wf * x;
          s2 += wf * (x - c) * (x - c);
        }
      }
    }
    if (mass) *mass = s0;
    if (first) *first = s1;
    if (sqerr) *sqerr = s2;
  }
};

// Symmetric Lloyd-Max on the positive half: boundaries 0, midpoints, 1; centroid of each
// cell = its conditional mean; iterate to the float64 fixed point.
static void solve_lloyd_max(int d, int bits, Codebook& out) {
  SphereDensity f(d);
  CellIntegrator ci(f, 48, 8);
  const int L = 1 << bits, h = L / 2;
  std::vector<double> c(h), nc(h), t(h + 1);
  double span = std::min(3.0 * f.sigma, 0.9);
  for (int k = 0; k < h; ++k) c[k] = (k + 0.5) * span / h;
  double prev = INFINITY;
  int stall = 0;
  for (int it = 0; it < 200000; ++it) {
    t[0] = 0.0;
    t[h] = 1.0;
    for (int k = 1; k < h; ++k) t[k] = 0.5 * (c[k - 1] + c[k]);
    double step = 0.0;
    for (int k = 0; k < h; ++k) {
      double m0, m1;
      ci.integrate(t[k], t[k + 1], 0.0, &m0, &m1, nullptr);
      nc[k] = m1 / m0;
      step = std::max(step, std::fabs(nc[k] - c[k]));
    }
    c.swap(nc);
    if (step == 0.0) break;
    if (step >= prev && step < 1e-14 * f.sigma) {
      if (++stall >= 3) break;
    }
    prev = step;
  }
  out.d = d;
  out.bits = bits;
  out.centroids.resize(L);
  out.thresholds.resize(L - 1);
  for (int k = 0; k < h; ++k) {
    out.centroids[h + k] = c[k];
    out.centroids[h - 1 - k] = -c[k];
  }
  for (int k = 0; k < L - 1; ++k) out.thresholds[k] = 0.5 * (out.centroids[k] + out.centroids[k + 1]);
  out.thresholds[h - 1] = 0.0;
  double mse = 0.0;
  for (int k = 0; k < L; ++k) {
    double a = k == 0 ? -1.0 : out.thresholds[k - 1];
    double b = k == L - 1 ? 1.0 : out.thresholds[k];
    double e;
    ci.integrate(a, b, out.centroids[k], nullptr, nullptr, &e);
    mse += e;
  }
  out.mse = mse;
}

// ------------------------------------------------------------------------------------
// float -> bf16 / fp16 bit patterns, round to nearest even.
static uint16_t to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static float from_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}
static uint16_t to_f16(double v) {
  // IEEE binary16 with round to nearest even, including subnormals (|v| < 65504 assumed)
  uint16_t sign = std::signbit(v) ? 0x8000 : 0;
  double a = std::fabs(v);
  if (a == 0.0) return sign;
  int e;
  double m = std::frexp(a, &e);  // a = m 2^e, m in [0.5, 1)
  int exp16 = e - 1 + 15;        // biased exponent of 1.xxx form
  if (exp16 >= 31) return sign | 0x7c00;
  double scaled;
  int biased;
  if (exp16 <= 0) {  // subnormal: units of 2^-24
    scaled = a * 16777216.0;
    biased = 0;
  } else {
    scaled = (m * 2.0 - 1.0) * 1024.0;  // fraction bits
    biased = exp16;
  }
  double fl = std::floor(scaled);
  double r = scaled - fl;
  uint32_t q = (uint32_t)fl;
  if (r > 0.5 || (r == 0.5 && (q & 1u))) ++q;
  uint32_t bitsv;
  if (biased == 0) {
    bitsv = q;  // may round up into the smallest normal, which the encoding absorbs
  } else {
    bitsv = ((uint32_t)biased << 10) + q;  // carry from q == 1024 bumps the exponent
  }
  if (bitsv >= 0x7c00u) return sign | 0x7c00;
  return sign | (uint16_t)bitsv;
}

static double from_f16(uint16_t h) {
  const int e = (h >> 10) & 31, m = h & 1023;
  double v = e == 0 ? std::ldexp((double)m, -24) : std::ldexp(1.0 + m / 1024.0, e - 15);
  return (h & 0x8000) ? -v : v;
}

// Relative error of rounding v > 0 (in fp16's normal range) to fp16: 11 significant bits,
// round to nearest even.
static double f16_rel_err(double v) {
  int e;
  const double x = std::ldexp(std::frexp(v, &e), 11);   // in [1024, 2048)
  return std::fabs(x - std::nearbyint(x)) / x;
}

// The decode's single-operand table holds 2^8 alpha c_k in fp16 and scales the result by
// 1 / alpha. The centroids are +-m_1 .. +-m_h (h = 2^(bits-1) magnitudes), so the table's
// worst relative error is the largest over the m_j; scanning alpha over 2^20 steps of [1, 2)
// (a power of two changes no relative error) finds one that leaves every m_j close to an
// fp16 value: about 1e-6 for two magnitudes, 2e-5 for four, 1e-4 for eight.
static void choose_decode_scale(Codebook& cb) {
  const int L = (int)cb.centroids.size(), h = L / 2;
  std::vector<double> m;
  for (int k = h; k < L; ++k) m.push_back(256.0 * cb.centroids[k]);
  // the largest magnitude first: fewest alphas survive it, so the scan stops early for most
  std::sort(m.begin(), m.end(), [](double a, double b) { return a > b; });
  double best = INFINITY, best_alpha = 1.0;
  // only codebooks that can take the table are scanned (alpha = 1 for the others)
  const int steps = h <= 4 ? 1 << 20 : 1;
  for (int i = 0; i < steps; ++i) {
    const double alpha = 1.0 + std::ldexp((double)i, -20);
    double worst = 0.0;
    for (double mj : m) {
      worst = std::max(worst, f16_rel_err(alpha * mj));
      if (worst >= best) break;
    }
    if (worst < best) {
      best = worst;
      best_alpha = alpha;
    }
  }
  cb.dec_alpha = best_alpha;
  // the bound from the table the kernels actually get
  double rho = 0.0;
  for (int k = 0; k < L; ++k) {
    const double v = 256.0 * best_alpha * cb.centroids[k];
    rho = std::max(rho, std::fabs(from_f16(to_f16(v)) - v) / std::fabs(v));
  }
  cb.dec_rho = rho;
}

LevelArgs make_levels(const Codebook& cb) {
  LevelArgs lv;
  std::memset(&lv, 0, sizeof(lv));
  const int L = 1 << cb.bits, h = L / 2;
  for (int j = 0; j < h - 1; ++j) lv.pos_thresholds[j] = (float)cb.thresholds[h + j];
  for (int j = h - 1; j < kMaxLevels / 2; ++j) lv.pos_thresholds[j] = INFINITY;
  for (int k = 0; k < L; ++k) {
    lv.centroid_f16[k] = to_f16(cb.centroids[k]);
    // decode operands c = c_hi + c_lo, both scaled by 2^8 so that c_lo stays a normal fp16 number
    const double chi = from_f16(lv.centroid_f16[k]);
    lv.dec_c_hi[k] = to_f16(256.0 * chi);
    lv.dec_c_lo[k] = to_f16(256.0 * (cb.centroids[k] - chi));
    lv.dec_c_one[k] = to_f16(256.0 * cb.dec_alpha * cb.centroids[k]);
    lv.centroid_f32[k] = (float)cb.centroids[k];
    lv.centroid_sq[k] = (float)(cb.centroids[k] * cb.centroids[k]);
    const uint16_t hi = to_bf16((float)cb.centroids[k]);
    const uint16_t lo = to_bf16((float)(cb.centroids[k] - (double)from_bf16(hi)));
    lv.centroid_bf16x2[k] = (uint32_t)hi | ((uint32_t)lo << 16);
  }
  lv.dec_one_nscale = (float)(0x1p-19 / cb.dec_alpha);
  lv.dec_one_rho = (float)cb.dec_rho;
  // Quantization table: |y| <= 1 (and a little beyond, for rounding) onto f in [1, 2); the bins
  // are 1/128 wide in f, 0.0156 in y, narrower than the boundary gaps of every codebook the
  // kernels take (the closest are 0.016 apart, d = 256 at 4 bits); checked below.
  lv.lut.scale = 0.5f * (1.0f - 0x1p-10f);
  lv.lut.offset = 1.5f;
  lv.lut.ok = true;
  float fthr[kMaxLevels];
  for (int k = 0; k < L - 1; ++k) fthr[k] = (float)(cb.thresholds[k] * (double)lv.lut.scale + 1.5);
  for (int j = 0; j < kLutBins; ++j) {
    const float lo = 1.0f + (float)j / 128.0f, hi = 1.0f + (float)(j + 1) / 128.0f;
    int nb = 0;
    float thr = 0.f;
    uint32_t base = 0;
    for (int k = 0; k < L - 1; ++k) {
      if (fthr[k] < lo) ++base;
      else if (fthr[k] < hi) {
        thr = fthr[k];
        ++nb;
      }
    }
    if (nb > 1) lv.lut.ok = false;
    const int top = 32 - cb.bits;   // carry position of entry_top (bits <= 8, so top >= 24)
    uint32_t e, et;
    if (nb) {
      std::memcpy(&e, &thr, 4);
      et = e + 1u - (1u << top) - (base << top);
      e = e + 1u - (1u << 24) - (base << 24);
    } else {
      std::memcpy(&e, &lo, 4);
      et = e - (base << top);
      e -= base << 24;
    }
    lv.lut.entry[j] = e;
    lv.lut.entry_top[j] = et;
  }
  return lv;
}


// ------------------------------------------------------------------------------------
// Householder QR of a d x d matrix (row-major) in float64; Q returned row-major.
static void householder_qr(int d, const double* g, std::vector<double>& q, std::vector<double>& r) {
  r.assign(g, g + (size_t)d * d);
  q.assign((size_t)d * d, 0.0);
  for (int i = 0; i < d; ++i) q[(size_t)i * d + i] = 1.0;
  std::vector<double> v(d), tmp(d);
  for (int k = 0; k < d - 1; ++k) {
    double norm = 0.0;
    for (int i = k; i < d; ++i) norm += r[(size_t)i * d + k] * r[(size_t)i * d + k];
    norm = std::sqrt(norm);
    if (norm == 0.0) continue;
    double x0 = r[(size_t)k * d + k];
    double alpha = x0 >= 0 ? -norm : norm;
    double vn = 0.0;
    for (int i = k; i < d; ++i) {
      v[i] = r[(size_t)i * d + k] - (i == k ? alpha : 0.0);
      vn += v[i] * v[i];
    }
    vn = std::sqrt(vn);
    if (vn == 0.0) continue;
    for (int i = k; i < d; ++i) v[i] /= vn;
    // R <- (I - 2 v v^T) R on rows k..d-1
    for (int j = 0; j < d; ++j) {
      double s = 0.0;
      for (int i = k; i < d; ++i) s += v[i] * r[(size_t)i * d + j];
      tmp[j] = 2.0 * s;
    }
    for (int i = k; i < d; ++i)
      for (int j = 0; j < d; ++j) r[(size_t)i * d + j] -= v[i] * tmp[j];
    // Q <- Q (I - 2 v v^T) on columns k..d-1
    for (int i = 0; i < d; ++i) {
      double s = 0.0;
      for (int j = k; j < d; ++j) s += q[(size_t)i * d + j] * v[j];
      s *= 2.0;
      for (int j = k; j < d; ++j) q[(size_t)i * d + j] -= s * v[j];
    }
  }
}

// Pi = Q diag(sign(diag R)) for G = Q R (G float32, promoted to float64), a zero sign
// counting as +1 (KV Cache API page, TurboQuantCompressorV2.__init__).
static void haar_from_gaussian(int d, const float* gaussian, double* pi) {
  const size_t dd = (size_t)d * d;
  std::vector<double> g(dd), q, r;
  for (size_t i = 0; i < dd; ++i) g[i] = (double)gaussian[i];
  householder_qr(d, g.data(), q, r);
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) {
      double s = r[(size_t)j * d + j] < 0 ? -1.0 : 1.0;
      pi[(size_t)i * d + j] = q[(size_t)i * d + j] * s;
    }
}

static double orthogonality_error(int d, const double* pi) {
  double worst = 0.0;
  for (int i = 0; i < d; ++i)
    for (int j = i; j < d; ++j) {
      double s = 0.0;
      for (int k = 0; k < d; ++k) s += pi[(size_t)k * d + i] * pi[(size_t)k * d + j];
      worst = std::max(worst, std::fabs(s - (i == j ? 1.0 : 0.0)));
    }
  return worst;
}

// MFMA A-operand tiles for the 32x32x16 (bf16/fp16) instructions. Tile (t, kb) of a matrix
// M is 64 lanes x 8 elements: lane l = m + 32*hh supplies M[sigma_t(m)][col(kb, hh) + e],
// e = 0..7, where output row sigma_t(m) = hh(m)*d/2 + 16 t + i(m), hh(m) = (m/4)%2,
// i(m) = 4*(m/8) + m%4. With that row order the 32x32 result lands so that lane
// (vector v, half hh) holds outputs hh*d/2 + 16 t + i in accumulator register i.
// Column order: col = hh*d/2 + 8 kb matches B operands taken from such accumulators (decode,
// the QJL sketch); with `paired`, col = 16 kb + 8 hh matches B operands loaded from memory
// (the encodes), where lanes v and v + 32 then read the two halves of one 32-byte piece.
template <typename F>
static void build_tiles(int d, F value, uint16_t* dst, bool paired = false) {
  const int T = d / 32, KB = d / 16, half = d / 2;
  for (int t = 0; t < T; ++t)
    for (int kb = 0; kb < KB; ++kb)
      for (int lane = 0; lane < 64; ++lane) {
        int m = lane % 32, hh = lane / 32;
        int row = ((m / 4) % 2) * half + 16 * t + 4 * (m / 8) + m % 4;
        for (int e = 0; e < 8; ++e) {
          int col = (paired ? 16 * kb + 8 * hh : hh * half + 8 * kb) + e;
          dst[(((size_t)t * KB + kb) * 64 + lane) * 8 + e] = value(row, col);
        }
      }
}

// Decode tiles of Pi^T: as build_tiles (column order hh*d/2 + 8 kb, the B operands come from a
// lane's packed chunk), with the output coordinates cut into qs slices of d/qs: slice q's tiles
// t' = 0 .. T/qs - 1 come first, and lane (vector v, half hh) ends up holding the slice
// coordinates q*d/qs + 32 t' + 16 hh + i in accumulator register i (a tile covers 32
// consecutive coordinates, so pairs of tiles give whole 128-byte pieces of a 16-bit row). Each slice holds two
// sets, `value(row, col, set)` for set 0 then set 1.
template <typename F>
static void build_dec_tiles(int d, int qs, F value, uint16_t* dst) {
  const int T = d / 32, KB = d / 16, TS = T / qs, sc = d / qs;
  size_t o = 0;
  for (int q = 0; q < qs; ++q)
    for (int set = 0; set < 2; ++set)
      for (int t = 0; t < TS; ++t)
        for (int kb = 0; kb < KB; ++kb)
          for (int lane = 0; lane < 64; ++lane) {
            const int m = lane % 32, hh = lane / 32;
            const int row = q * sc + 32 * t + 16 * ((m / 4) % 2) + 4 * (m / 8) + m % 4;
            for (int e = 0; e < 8; ++e) dst[o++] = value(row, hh * (d / 2) + 8 * kb + e, set);
          }
}

static int upload_rotation(Rotation& R) {
  int dev = 0, count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0)
    return fail(TQ_ERR_NO_DEVICE, "tq_rotation: no HIP device is available");
  if (hipGetDevice(&dev) != hipSuccess) return fail(TQ_ERR_NO_DEVICE, "tq_rotation: hipGetDevice failed");
  const int d = R.d;
  const size_t dd = (size_t)d * d;
  R.enc_stride = 4 * dd;
  R.dec_stride = 4 * dd;
  R.f32_stride = 4 * dd;
  R.enc_off = 0;
  R.dec_off = R.enc_stride * R.n_rot;
  R.f32_off = R.dec_off + R.dec_stride * R.n_rot;
  R.f32t_off = R.f32_off + R.f32_stride * R.n_rot;
  R.pad_off = R.f32t_off + R.f32_stride * R.n_rot;
  size_t total = R.pad_off + Rotation::kZeroBytes + Rotation::kSinkBytes;
  std::vector<uint8_t> host(total);   // the zero page and sink upload as zeros
  for (int r = 0; r < R.n_rot; ++r) {
    const double* P = R.pi.data() + (size_t)r * dd;
    uint16_t* hi = (uint16_t*)(host.data() + R.enc_off + r * R.enc_stride);
    uint16_t* lo = hi + dd;
    // encode: y = Pi x, tiles of Pi split as bf16 hi + bf16 lo
    build_tiles(d, [&](int row, int col) { return to_bf16((float)P[(size_t)row * d + col]); }, hi, true);
    build_tiles(d, [&](int row, int col) {
      double v = P[(size_t)row * d + col];
      float h = from_bf16(to_bf16((float)v));
      return to_bf16((float)(v - (double)h));
    }, lo, true);
    // decode: x = Pi^T c, tiles of 2^11 P_hi and 2^11 P_lo with Pi^T = P_hi + P_lo in fp16
    uint16_t* de = (uint16_t*)(host.data() + R.dec_off + r * R.dec_stride);
    build_dec_tiles(d, d == 256 ? 4 : 1, [&](int row, int col, int set) {
      const double v = P[(size_t)col * d + row];
      const double hi = from_f16(to_f16(v));
      return to_f16(2048.0 * (set == 0 ? hi : v - hi));
    }, de);
    float* f = (float*)(host.data() + R.f32_off + r * R.f32_stride);
    for (size_t i = 0; i < dd; ++i) f[i] = (float)P[i];
    float* ft = (float*)(host.data() + R.f32t_off + r * R.f32_stride);
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j) ft[(size_t)j * d + i] = (float)P[(size_t)i * d + j];
  }
  hipError_t e = hipMalloc(&R.dev, total);
  if (e != hipSuccess) return fail(TQ_ERR_HIP, std::string("tq_rotation: hipMalloc: ") + hipGetErrorString(e));
  e = hipMemcpy(R.dev, host.data(), total, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(R.dev);
    R.dev = nullptr;
    return fail(TQ_ERR_HIP, std::string("tq_rotation: hipMemcpy: ") + hipGetErrorString(e));
  }
  R.device = dev;
  return TQ_OK;
}

// QJL sketch upload: M_r = S_r Pi_r^T (float64 products of the float32 sketch and the float64
// rotation) as bf16 hi / lo tiles in Pi's encode tile order, and S_r^T in float32 for the
// query projection S q.
static int upload_qjl(Qjl& Q, const float* sketch) {
  const int d = Q.d;
  const size_t dd = (size_t)d * d;
  Q.frag_stride = 4 * dd;
  Q.st_stride = 4 * dd;
  Q.frag_off = 0;
  Q.st_off = Q.frag_stride * Q.n_rot;
  const size_t total = Q.st_off + Q.st_stride * Q.n_rot;
  std::vector<uint8_t> host(total);
  std::vector<double> m(dd);
  for (int r = 0; r < Q.n_rot; ++r) {
    const float* S = sketch + (size_t)r * dd;
    const double* P = Q.rot->pi.data() + (size_t)r * dd;
    for (int i = 0; i < d; ++i)
      for (int k = 0; k < d; ++k) {
        double acc = 0.0;
        for (int j = 0; j < d; ++j) acc += (double)S[(size_t)i * d + j] * P[(size_t)k * d + j];
        m[(size_t)i * d + k] = acc;
      }
    uint16_t* hi = (uint16_t*)(host.data() + Q.frag_off + r * Q.frag_stride);
    uint16_t* lo = hi + dd;
    build_tiles(d, [&](int row, int col) { return to_bf16((float)m[(size_t)row * d + col]); }, hi);
    build_tiles(d, [&](int row, int col) {
      double v = m[(size_t)row * d + col];
      float h = from_bf16(to_bf16((float)v));
      return to_bf16((float)(v - (double)h));
    }, lo);
    float* st = (float*)(host.data() + Q.st_off + r * Q.st_stride);
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j) st[(size_t)j * d + i] = S[(size_t)i * d + j];
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(TQ_ERR_NO_DEVICE, "tq_qjl_create: hipGetDevice failed");
  if (dev != Q.rot->device)
    return fail(TQ_ERR_NO_DEVICE, "tq_qjl_create: the rotation lives on device " + std::to_string(Q.rot->device) +
                                      " but device " + std::to_string(dev) + " is current");
  hipError_t e = hipMalloc(&Q.dev, total);
  if (e != hipSuccess) return fail(TQ_ERR_HIP, std::string("tq_qjl_create: hipMalloc: ") + hipGetErrorString(e));
  e = hipMemcpy(Q.dev, host.data(), total, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(Q.dev);
    Q.dev = nullptr;
    return fail(TQ_ERR_HIP, std::string("tq_qjl_create: hipMemcpy: ") + hipGetErrorString(e));
  }
  Q.device = dev;
  return TQ_OK;
}

hipError_t set_kernel_lds(const void* kernel, int device, size_t lds) {
  static std::mutex mu;
  static std::set<std::pair<const void*, int>> done;
  std::lock_guard<std::mutex> lk(mu);
  if (done.count({kernel, device})) return hipSuccess;
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (cur != device) (void)hipSetDevice(cur);
  if (e == hipSuccess) done.insert({kernel, device});
  return e;
}

int device_cu_count(int device) {
  static int cached[64] = {0};
  if (device >= 0 && device < 64 && cached[device]) return cached[device];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || n <= 0) n = 256;
  if (device >= 0 && device < 64) cached[device] = n;
  return n;
}

}  // namespace tq

using namespace tq;

static bool gpu_dim_ok(int d) { return d == 64 || d == 128 || d == 256; }
static bool gpu_bits_ok(int b) { return b >= 2 && b <= 4; }
static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

static int check_device(const Rotation& R, const char* who) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess)
    return fail(TQ_ERR_NO_DEVICE, std::string(who) + ": hipGetDevice failed");
  if (dev != R.device)
    return fail(TQ_ERR_NO_DEVICE, std::string(who) + ": the rotation was created on device " +
                                      std::to_string(R.device) + " but device " + std::to_string(dev) +
                                      " is current");
  return TQ_OK;
}

static int hip_status(hipError_t e, const char* who) {
  if (e == hipSuccess) return TQ_OK;
  return fail(TQ_ERR_HIP, std::string(who) + ": kernel launch failed: " + hipGetErrorString(e));
}

extern "C" {

int tq_version(void) { return TQ_VERSION; }

const char* tq_last_error(void) { return g_error.c_str(); }

tq_codebook_t* tq_codebook_init(int d, int bits) {
  if (d < 3 || d > 4096) {
    set_error("tq_codebook_init: d = " + std::to_string(d) + " is out of range; accepted 3..4096");
    return nullptr;
  }
  if (bits < 1 || bits > 4) {
    set_error("tq_codebook_init: bits = " + std::to_string(bits) + " is out of range; accepted 1..4");
    return nullptr;
  }
  tq_codebook_t* h = new tq_codebook_t;
  solve_lloyd_max(d, bits, h->cb);
  choose_decode_scale(h->cb);
  set_error("");
  return h;
}

int tq_codebook_get(const tq_codebook_t* cb, double* centroids, double* thresholds, double* mse) {
  if (!cb) return fail(TQ_ERR_NULL, "tq_codebook_get: cb is NULL");
  if (centroids) std::copy(cb->cb.centroids.begin(), cb->cb.centroids.end(), centroids);
  if (thresholds) std::copy(cb->cb.thresholds.begin(), cb->cb.thresholds.end(), thresholds);
  if (mse) *mse = cb->cb.mse;
  return TQ_OK;
}

int tq_codebook_dims(const tq_codebook_t* cb, int* d, int* bits) {
  if (!cb) return fail(TQ_ERR_NULL, "tq_codebook_dims: cb is NULL");
  if (d) *d = cb->cb.d;
  if (bits) *bits = cb->cb.bits;
  return TQ_OK;
}

void tq_codebook_free(tq_codebook_t* cb) { delete cb; }

static tq_rotation_t* make_rotation(int d, int n_rot, std::vector<double>&& pi, bool hadamard = false) {
  tq_rotation_t* h = new tq_rotation_t;
  h->rot.d = d;
  h->rot.n_rot = n_rot;
  h->rot.hadamard = hadamard;
  h->rot.pi = std::move(pi);
  if (upload_rotation(h->rot) != TQ_OK) {
    delete h;
    return nullptr;
  }
  set_error("");
  return h;
}

tq_rotation_t* tq_rotation_from_gaussian(int d, int n_rot, const float* gaussian) {
  if (!gpu_dim_ok(d)) {
    set_error("tq_rotation_from_gaussian: d = " + std::to_string(d) + " is not supported; accepted 64, 128, 256");
    return nullptr;
  }
  if (n_rot < 1 || n_rot > 65535) {
    set_error("tq_rotation_from_gaussian: n_rot = " + std::to_string(n_rot) + " is out of range; accepted 1..65535");
    return nullptr;
  }
  if (!gaussian) {
    set_error("tq_rotation_from_gaussian: gaussian is NULL");
    return nullptr;
  }
  const size_t dd = (size_t)d * d;
  std::vector<double> pi(dd * n_rot);
  for (int k = 0; k < n_rot; ++k) haar_from_gaussian(d, gaussian + k * dd, pi.data() + k * dd);
  return make_rotation(d, n_rot, std::move(pi));
}

int tq_rotation_compute(int d, const float* gaussian, double* pi) {
  if (d < 3 || d > 4096)
    return fail(TQ_ERR_INVALID_ARG, "tq_rotation_compute: d = " + std::to_string(d) + " is out of range; accepted 3..4096");
  if (!gaussian) return fail(TQ_ERR_NULL, "tq_rotation_compute: gaussian is NULL");
  if (!pi) return fail(TQ_ERR_NULL, "tq_rotation_compute: pi is NULL");
  haar_from_gaussian(d, gaussian, pi);
  return TQ_OK;
}

tq_rotation_t* tq_rotation_from_matrix(int d, int n_rot, const double* pi_in) {
  if (!gpu_dim_ok(d)) {
    set_error("tq_rotation_from_matrix: d = " + std::to_string(d) + " is not supported; accepted 64, 128, 256");
    return nullptr;
  }
  if (n_rot < 1 || n_rot > 65535) {
    set_error("tq_rotation_from_matrix: n_rot = " + std::to_string(n_rot) + " is out of range; accepted 1..65535");
    return nullptr;
  }
  if (!pi_in) {
    set_error("tq_rotation_from_matrix: pi is NULL");
    return nullptr;
  }
  const size_t dd = (size_t)d * d;
  for (int k = 0; k < n_rot; ++k) {
    double err = orthogonality_error(d, pi_in + k * dd);
    if (!(err <= 1e-9)) {
      char buf[160];
      std::snprintf(buf, sizeof(buf),
                    "tq_rotation_from_matrix: rotation %d is not orthogonal (max|Pi^T Pi - I| = %.3g > 1e-9)",
                    k, err);
      set_error(buf);
      return nullptr;
    }
  }
  std::vector<double> pi(pi_in, pi_in + dd * n_rot);
  return make_rotation(d, n_rot, std::move(pi));
}

tq_rotation_t* tq_rotation_hadamard(int d, int n_rot, const int8_t* signs) {
  if (!gpu_dim_ok(d)) {
    set_error("tq_rotation_hadamard: d = " + std::to_string(d) + " is not supported; accepted 64, 128, 256");
    return nullptr;
  }
  if (n_rot < 1 || n_rot > 65535) {
    set_error("tq_rotation_hadamard: n_rot = " + std::to_string(n_rot) + " is out of range; accepted 1..65535");
    return nullptr;
  }
  const size_t dd = (size_t)d * d;
  if (signs) {
    for (size_t i = 0; i < (size_t)n_rot * d; ++i)
      if (signs[i] != 1 && signs[i] != -1) {
        set_error("tq_rotation_hadamard: signs[" + std::to_string(i) + "] = " + std::to_string((int)signs[i]) +
                  "; accepted +1 or -1");
        return nullptr;
      }
  }
  // Pi[i][j] = (-1)^popcount(i & j) * s_j / sqrt(d): Sylvester's Walsh-Hadamard matrix with a
  // sign per input channel, orthonormal
  const double inv = 1.0 / std::sqrt((double)d);
  std::vector<double> pi(dd * n_rot);
  for (int r = 0; r < n_rot; ++r)
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j) {
        const double h = (__builtin_popcount((unsigned)(i & j)) & 1) ? -inv : inv;
        const double sj = signs ? (double)signs[(size_t)r * d + j] : 1.0;
        pi[(size_t)r * dd + (size_t)i * d + j] = h * sj;
      }
  return make_rotation(d, n_rot, std::move(pi), true);
}

int tq_rotation_get(const tq_rotation_t* rot, double* pi) {
  if (!rot) return fail(TQ_ERR_NULL, "tq_rotation_get: rot is NULL");
  if (!pi) return fail(TQ_ERR_NULL, "tq_rotation_get: pi is NULL");
  std::copy(rot->rot.pi.begin(), rot->rot.pi.end(), pi);
  return TQ_OK;
}

int tq_rotation_dims(const tq_rotation_t* rot, int* d, int* n_rot) {
  if (!rot) return fail(TQ_ERR_NULL, "tq_rotation_dims: rot is NULL");
  if (d) *d = rot->rot.d;
  if (n_rot) *n_rot = rot->rot.n_rot;
  return TQ_OK;
}

void tq_rotation_free(tq_rotation_t* rot) {
  if (!rot) return;
  if (rot->rot.dev) (void)hipFree(rot->rot.dev);
  delete rot;
}

static int dtype_size(int dt) { return dt == TQ_F32 ? 4 : (dt == TQ_BF16 || dt == TQ_F16) ? 2 : 0; }

static int check_pair(const tq_codebook_t* cb, const tq_rotation_t* rot, const char* who) {
  if (!cb) return fail(TQ_ERR_NULL, std::string(who) + ": cb is NULL");
  if (!rot) return fail(TQ_ERR_NULL, std::string(who) + ": rot is NULL");
  if (!gpu_bits_ok(cb->cb.bits))
    return fail(TQ_ERR_INVALID_ARG, std::string(who) + ": codebook bits = " + std::to_string(cb->cb.bits) +
                                        " is not supported on the GPU; accepted 2, 3, 4");
  if (cb->cb.d != rot->rot.d)
    return fail(TQ_ERR_INVALID_ARG, std::string(who) + ": codebook d = " + std::to_string(cb->cb.d) +
                                        " does not match rotation d = " + std::to_string(rot->rot.d));
  return TQ_OK;
}

static int check_rot_index(int64_t n, int64_t vpr, int n_rot, const char* who) {
  if (vpr < 0) return fail(TQ_ERR_INVALID_ARG, std::string(who) + ": vectors_per_rot must be >= 0");
  if (vpr > 0 && n > 0) {
    int64_t need = (n + vpr - 1) / vpr;
    if (need > n_rot)
      return fail(TQ_ERR_INVALID_ARG, std::string(who) + ": n / vectors_per_rot needs " + std::to_string(need) +
                                          " rotations but the stack has " + std::to_string(n_rot));
  }
  return TQ_OK;
}

static int encode_impl(const char* who, bool norm_correct, const tq_codebook_t* cb, const tq_rotation_t* rot,
                       int64_t vectors_per_rot, const void* x, int x_dtype, int64_t n, int64_t x_row_stride,
                       uint8_t* packed, float* norms, const int64_t* slot_mapping, tq_stream_t stream) {
  const std::string W(who);
  int s = check_pair(cb, rot, who);
  if (s) return s;
  const int d = rot->rot.d;
  if (n < 0) return fail(TQ_ERR_INVALID_ARG, W + ": n must be >= 0");
  int es = dtype_size(x_dtype);
  if (!es) return fail(TQ_ERR_INVALID_ARG, W + ": x_dtype = " + std::to_string(x_dtype) +
                                               " is not supported; accepted TQ_F32 (0), TQ_BF16 (1), TQ_F16 (2)");
  if (x_row_stride < d)
    return fail(TQ_ERR_INVALID_ARG, W + ": x_row_stride = " + std::to_string(x_row_stride) +
                                        " is smaller than d = " + std::to_string(d));
  if ((s = check_rot_index(n, vectors_per_rot, rot->rot.n_rot, who))) return s;
  if (n == 0) return TQ_OK;
  if (!x) return fail(TQ_ERR_NULL, W + ": x is NULL");
  if (!packed) return fail(TQ_ERR_NULL, W + ": packed is NULL");
  if (!norms) return fail(TQ_ERR_NULL, W + ": norms is NULL");
  if (!aligned(x, 16)) return fail(TQ_ERR_ALIGN, W + ": x must be 16-byte aligned");
  if ((x_row_stride * es) % 16) return fail(TQ_ERR_ALIGN, W + ": x_row_stride * element size must be a multiple of 16 bytes");
  if (!aligned(packed, 8)) return fail(TQ_ERR_ALIGN, W + ": packed must be 8-byte aligned");
  if (!aligned(norms, 4)) return fail(TQ_ERR_ALIGN, W + ": norms must be 4-byte aligned");
  if (slot_mapping && !aligned(slot_mapping, 8)) return fail(TQ_ERR_ALIGN, W + ": slot_mapping must be 8-byte aligned");
  if ((s = check_device(rot->rot, who))) return s;
  EncodeLaunch a;
  a.rot = &rot->rot;
  a.lv = make_levels(cb->cb);
  if (!lut_covers_unit_range(a.lv))
    return fail(TQ_ERR_INVALID_ARG, W + ": the codebook's boundaries are too close for the quantization table");
  a.bits = cb->cb.bits;
  a.x_dtype = x_dtype;
  a.vectors_per_rot = vectors_per_rot;
  a.n = n;
  a.x_row_stride = x_row_stride;
  a.x = x;
  a.packed = packed;
  a.norms = norms;
  a.slot_mapping = slot_mapping;
  a.norm_correct = norm_correct;
  a.stream = (hipStream_t)stream;
  return hip_status(launch_encode(a), who);
}

int tq_encode(const tq_codebook_t* cb, const tq_rotation_t* rot, int64_t vectors_per_rot, const void* x,
              int x_dtype, int64_t n, int64_t x_row_stride, uint8_t* packed, float* norms,
              const int64_t* slot_mapping, tq_stream_t stream) {
  return encode_impl("tq_encode", false, cb, rot, vectors_per_rot, x, x_dtype, n, x_row_stride, packed, norms,
                     slot_mapping, stream);
}

int tq_encode_norm_corrected(const tq_codebook_t* cb, const tq_rotation_t* rot, int64_t vectors_per_rot,
                             const void* x, int x_dtype, int64_t n, int64_t x_row_stride, uint8_t* packed,
                             float* norms, const int64_t* slot_mapping, tq_stream_t stream) {
  return encode_impl("tq_encode_norm_corrected", true, cb, rot, vectors_per_rot, x, x_dtype, n, x_row_stride,
                     packed, norms, slot_mapping, stream);
}

tq_qjl_t* tq_qjl_create(const tq_rotation_t* rot, const float* sketch) {
  if (!rot) {
    set_error("tq_qjl_create: rot is NULL");
    return nullptr;
  }
  if (!sketch) {
    set_error("tq_qjl_create: sketch is NULL");
    return nullptr;
  }
  if (!gpu_dim_ok(rot->rot.d)) {
    set_error("tq_qjl_create: d = " + std::to_string(rot->rot.d) + " is not supported; accepted 64, 128, 256");
    return nullptr;
  }
  const size_t dd = (size_t)rot->rot.d * rot->rot.d;
  for (size_t i = 0; i < dd * rot->rot.n_rot; ++i)
    if (!std::isfinite(sketch[i])) {
      set_error("tq_qjl_create: sketch has a non-finite entry at index " + std::to_string(i));
      return nullptr;
    }
  tq_qjl_t* h = new tq_qjl_t;
  h->q.rot = &rot->rot;
  h->q.d = rot->rot.d;
  h->q.n_rot = rot->rot.n_rot;
  if (upload_qjl(h->q, sketch) != TQ_OK) {
    delete h;
    return nullptr;
  }
  set_error("");
  return h;
}

void tq_qjl_free(tq_qjl_t* qjl) {
  if (!qjl) return;
  if (qjl->q.dev) (void)hipFree(qjl->q.dev);
  delete qjl;
}

int tq_qjl_encode(const tq_codebook_t* cb, const tq_qjl_t* qjl, int64_t vectors_per_rot, const void* x,
                  int x_dtype, int64_t n, int64_t x_row_stride, uint8_t* packed, float* norms, uint8_t* signs,
                  float* rnorms, const int64_t* slot_mapping, tq_stream_t stream) {
  const char* who = "tq_qjl_encode";
  const std::string W(who);
  if (!qjl) return fail(TQ_ERR_NULL, W + ": qjl is NULL");
  const Rotation& R = *qjl->q.rot;
  if (!cb) return fail(TQ_ERR_NULL, W + ": cb is NULL");
  if (cb->cb.bits < 1 || cb->cb.bits > 4)
    return fail(TQ_ERR_INVALID_ARG, W + ": codebook bits = " + std::to_string(cb->cb.bits) +
                                        " is not supported on the GPU; accepted 1..4 (keys of 2..5 bits)");
  if (cb->cb.d != R.d)
    return fail(TQ_ERR_INVALID_ARG, W + ": codebook d = " + std::to_string(cb->cb.d) + " does not match d = " +
                                        std::to_string(R.d));
  if (n < 0) return fail(TQ_ERR_INVALID_ARG, W + ": n must be >= 0");
  const int es = dtype_size(x_dtype);
  if (!es) return fail(TQ_ERR_INVALID_ARG, W + ": x_dtype = " + std::to_string(x_dtype) +
                                               " is not supported; accepted TQ_F32 (0), TQ_BF16 (1), TQ_F16 (2)");
  if (x_row_stride < R.d)
    return fail(TQ_ERR_INVALID_ARG, W + ": x_row_stride = " + std::to_string(x_row_stride) +
                                        " is smaller than d = " + std::to_string(R.d));
  int s = check_rot_index(n, vectors_per_rot, R.n_rot, who);
  if (s) return s;
  if (n == 0) return TQ_OK;
  if (!x) return fail(TQ_ERR_NULL, W + ": x is NULL");
  if (!packed || !norms || !signs || !rnorms) return fail(TQ_ERR_NULL, W + ": an output pointer is NULL");
  if (!aligned(x, 16)) return fail(TQ_ERR_ALIGN, W + ": x must be 16-byte aligned");
  if ((x_row_stride * es) % 16) return fail(TQ_ERR_ALIGN, W + ": x_row_stride * element size must be a multiple of 16 bytes");
  if (!aligned(packed, 8)) return fail(TQ_ERR_ALIGN, W + ": packed must be 8-byte aligned");
  if (!aligned(norms, 4) || !aligned(rnorms, 4)) return fail(TQ_ERR_ALIGN, W + ": norms / rnorms must be 4-byte aligned");
  if (!aligned(signs, 16)) return fail(TQ_ERR_ALIGN, W + ": signs must be 16-byte aligned");
  if (slot_mapping && !aligned(slot_mapping, 8)) return fail(TQ_ERR_ALIGN, W + ": slot_mapping must be 8-byte aligned");
  if ((s = check_device(R, who))) return s;
  QjlEncodeLaunch q;
  EncodeLaunch& a = q.enc;
  a.rot = &R;
  a.lv = make_levels(cb->cb);
  if (!lut_covers_unit_range(a.lv))
    return fail(TQ_ERR_INVALID_ARG, W + ": the codebook's boundaries are too close for the quantization table");
  a.bits = cb->cb.bits;
  a.x_dtype = x_dtype;
  a.vectors_per_rot = vectors_per_rot;
  a.n = n;
  a.x_row_stride = x_row_stride;
  a.x = x;
  a.packed = packed;
  a.norms = norms;
  a.slot_mapping = slot_mapping;
  a.norm_correct = false;
  a.stream = (hipStream_t)stream;
  q.qjl = &qjl->q;
  q.signs = signs;
  q.rnorms = rnorms;
  return hip_status(launch_qjl_encode(q), who);
}

int tq_decode(const tq_codebook_t* cb, const tq_rotation_t* rot, int64_t vectors_per_rot, const uint8_t* packed,
              const float* norms, const int64_t* slot_mapping, int64_t n, void* out, int out_dtype,
              tq_stream_t stream) {
  int s = check_pair(cb, rot, "tq_decode");
  if (s) return s;
  if (n < 0) return fail(TQ_ERR_INVALID_ARG, "tq_decode: n must be >= 0");
  if (!dtype_size(out_dtype))
    return fail(TQ_ERR_INVALID_ARG, "tq_decode: out_dtype = " + std::to_string(out_dtype) +
                                        " is not supported; accepted TQ_F32 (0), TQ_BF16 (1), TQ_F16 (2)");
  if ((s = check_rot_index(n, vectors_per_rot, rot->rot.n_rot, "tq_decode"))) return s;
  if (n == 0) return TQ_OK;
  if (!packed) return fail(TQ_ERR_NULL, "tq_decode: packed is NULL");
  if (!norms) return fail(TQ_ERR_NULL, "tq_decode: norms is NULL");
  if (!out) return fail(TQ_ERR_NULL, "tq_decode: out is NULL");
  if (!aligned(packed, 8)) return fail(TQ_ERR_ALIGN, "tq_decode: packed must be 8-byte aligned");
  if (!aligned(norms, 4)) return fail(TQ_ERR_ALIGN, "tq_decode: norms must be 4-byte aligned");
  if (!aligned(out, 16)) return fail(TQ_ERR_ALIGN, "tq_decode: out must be 16-byte aligned");
  if (slot_mapping && !aligned(slot_mapping, 8)) return fail(TQ_ERR_ALIGN, "tq_decode: slot_mapping must be 8-byte aligned");
  if ((s = check_device(rot->rot, "tq_decode"))) return s;
  if (!rot->rot.hadamard && decode_one_operand(cb->cb.bits, out_dtype) && cb->cb.dec_rho > kDecOneOperandRho)
    return fail(TQ_ERR_INVALID_ARG, "tq_decode: no fp16 table of this codebook's centroids is accurate enough "
                                    "for a bfloat16 decode (relative error " + std::to_string(cb->cb.dec_rho) + ")");
  DecodeLaunch a;
  a.rot = &rot->rot;
  a.lv = make_levels(cb->cb);
  a.bits = cb->cb.bits;
  a.out_dtype = out_dtype;
  a.vectors_per_rot = vectors_per_rot;
  a.n = n;
  a.packed = packed;
  a.norms = norms;
  a.slot_mapping = slot_mapping;
  a.out = out;
  a.stream = (hipStream_t)stream;
  return hip_status(launch_decode(a), "tq_decode");
}

static int check_attn(const tq_attn_params* p, bool scores_only, const char* who) {
  if (!p) return fail(TQ_ERR_NULL, std::string(who) + ": params is NULL");
  int s;
  if (p->qjl_k && p->cb_k && p->cb_k->cb.bits == 1) {
    // QJL keys of 2 bits: a 1-bit MSE stage under the sign sketch
    if (!p->rot_k) return fail(TQ_ERR_NULL, std::string(who) + ": rot_k is NULL");
    if (p->cb_k->cb.d != p->rot_k->rot.d)
      return fail(TQ_ERR_INVALID_ARG, std::string(who) + ": codebook d = " + std::to_string(p->cb_k->cb.d) +
                                          " does not match rotation d = " + std::to_string(p->rot_k->rot.d));
  } else if ((s = check_pair(p->cb_k, p->rot_k, who))) {
    return s;
  }
  if (!scores_only) {
    if ((s = check_pair(p->cb_v, p->rot_v, who))) return s;
    if (p->rot_v->rot.d != p->rot_k->rot.d)
      return fail(TQ_ERR_INVALID_ARG, std::string(who) + ": K and V rotations have different d");
    if (p->rot_v->rot.device != p->rot_k->rot.device)
      return fail(TQ_ERR_NO_DEVICE, std::string(who) + ": K and V rotations live on different devices");
  }
  if (p->batch < 0 || p->num_q_heads <= 0 || p->num_kv_heads <= 0)
    return fail(TQ_ERR_INVALID_ARG, std::string(who) + ": batch must be >= 0 and head counts > 0");
  if (p->num_q_heads % p->num_kv_heads)
    return fail(TQ_ERR_INVALID_ARG, std::string(who) + ": num_q_heads = " + std::to_string(p->num_q_heads) +
                                        " is not a multiple of num_kv_heads = " + std::to_string(p->num_kv_heads));
  int G = p->num_q_heads / p->num_kv_heads;
  if (G > 16)
    return fail(TQ_ERR_INVALID_ARG, std::string(who) + ": num_q_heads / num_kv_heads = " + std::to_string(G) +
                                        " is not supported; accepted 1..16");
  if (p->max_seq_len < 0) return fail(TQ_ERR_INVALID_ARG, std::string(who) + ": max_seq_len must be >= 0");
  if (!dtype_size(p->q_dtype))
    return fail(TQ_ERR_INVALID_ARG, std::string(who) + ": q_dtype is not supported; accepted TQ_F32, TQ_BF16, TQ_F16");
  if (!scores_only && !dtype_size(p->out_dtype))
    return fail(TQ_ERR_INVALID_ARG, std::string(who) + ": out_dtype is not supported; accepted TQ_F32, TQ_BF16, TQ_F16");
  if (p->batch_per_rot < 0) return fail(TQ_ERR_INVALID_ARG, std::string(who) + ": batch_per_rot must be >= 0");
  if (p->batch_per_rot > 0 && p->batch > 0) {
    int64_t need = ((int64_t)p->batch + p->batch_per_rot - 1) / p->batch_per_rot;
    if (need > p->rot_k->rot.n_rot || (!scores_only && need > p->rot_v->rot.n_rot))
      return fail(TQ_ERR_INVALID_ARG, std::string(who) + ": batch / batch_per_rot exceeds the rotation stack");
  }
  if (p->block_table) {
    if (p->block_size <= 0 || p->max_blocks_per_seq <= 0)
      return fail(TQ_ERR_INVALID_ARG, std::string(who) + ": paged layout needs block_size > 0 and max_blocks_per_seq > 0");
    if ((int64_t)p->block_size * p->max_blocks_per_seq < p->max_seq_len)
      return fail(TQ_ERR_INVALID_ARG, std::string(who) + ": block_size * max_blocks_per_seq < max_seq_len");
  }
  if (!p->block_table) {
    // dense caches are read through buffer resources with 32-bit byte offsets within one
    // (sequence, KV head)'s rows
    const int64_t d = p->rot_k->rot.d;
    int64_t row = d * p->cb_k->cb.bits / 8;
    if (!scores_only) row = std::max(row, d * (int64_t)p->cb_v->cb.bits / 8);
    if ((int64_t)p->max_seq_len * row >= ((int64_t)1 << 32))
      return fail(TQ_ERR_INVALID_ARG, std::string(who) + ": max_seq_len = " + std::to_string(p->max_seq_len) +
                                          " is too long for a dense cache (rows of one sequence and KV head must span"
                                          " less than 4 GiB); use the paged layout");
  }
  if (p->num_splits < 0) return fail(TQ_ERR_INVALID_ARG, std::string(who) + ": num_splits must be >= 0");
  if (p->window < 0) return fail(TQ_ERR_INVALID_ARG, std::string(who) + ": window must be >= 0");
  if (p->window > 0 && !scores_only) {
    const int es = dtype_size(p->window_dtype);
    if (!es)
      return fail(TQ_ERR_INVALID_ARG, std::string(who) + ": window_dtype is not supported; accepted TQ_F32, TQ_BF16, TQ_F16");
    if (p->batch > 0 && (!p->k_window || !p->v_window))
      return fail(TQ_ERR_NULL, std::string(who) + ": window > 0 needs k_window and v_window");
    if (!aligned(p->k_window, es) || !aligned(p->v_window, es))
      return fail(TQ_ERR_ALIGN, std::string(who) + ": k_window / v_window must be aligned to the element size");
  }
  if (p->qjl_k && p->qjl_k->q.rot != &p->rot_k->rot)
    return fail(TQ_ERR_INVALID_ARG, std::string(who) + ": qjl_k was not created on rot_k");
  return TQ_OK;
}

size_t tq_attn_workspace_size(const tq_attn_params* p) {
  if (check_attn(p, true, "tq_attn_workspace_size")) return 0;
  int dev = p->rot_k->rot.device;
  return attn_workspace_layout(p, p->rot_k->rot.d, device_cu_count(dev)).total;
}

static int attn_common(const tq_attn_params* p, float* scores, bool scores_only, tq_stream_t stream, const char* who,
                       bool static_scratch = false) {
  int s = check_attn(p, scores_only, who);
  if (s) return s;
  if (p->batch == 0 || p->max_seq_len == 0) {
    if (scores_only) return TQ_OK;
  }
  if (p->batch == 0) return TQ_OK;
  if (!p->q) return fail(TQ_ERR_NULL, std::string(who) + ": q is NULL");
  if (!aligned(p->q, 16)) return fail(TQ_ERR_ALIGN, std::string(who) + ": q must be 16-byte aligned");
  if (p->max_seq_len > 0) {
    if (!p->k_packed || !p->k_norms) return fail(TQ_ERR_NULL, std::string(who) + ": k_packed / k_norms is NULL");
    if (!aligned(p->k_packed, 8) || !aligned(p->k_norms, 4))
      return fail(TQ_ERR_ALIGN, std::string(who) + ": k_packed must be 8-byte and k_norms 4-byte aligned");
    if (p->qjl_k) {
      if (!p->k_signs || !p->k_rnorms) return fail(TQ_ERR_NULL, std::string(who) + ": qjl_k needs k_signs and k_rnorms");
      if (!aligned(p->k_signs, 16) || !aligned(p->k_rnorms, 4))
        return fail(TQ_ERR_ALIGN, std::string(who) + ": k_signs must be 16-byte and k_rnorms 4-byte aligned");
    }
    if (!scores_only) {
      if (!p->v_packed || !p->v_norms) return fail(TQ_ERR_NULL, std::string(who) + ": v_packed / v_norms is NULL");
      if (!aligned(p->v_packed, 8) || !aligned(p->v_norms, 4))
        return fail(TQ_ERR_ALIGN, std::string(who) + ": v_packed must be 8-byte and v_norms 4-byte aligned");
    }
  }
  if (scores_only) {
    if (!scores) return fail(TQ_ERR_NULL, std::string(who) + ": scores is NULL");
    if (!aligned(scores, 4)) return fail(TQ_ERR_ALIGN, std::string(who) + ": scores must be 4-byte aligned");
  } else {
    if (!p->out) return fail(TQ_ERR_NULL, std::string(who) + ": out is NULL");
    if (!aligned(p->out, 16)) return fail(TQ_ERR_ALIGN, std::string(who) + ": out must be 16-byte aligned");
  }
  const int d = p->rot_k->rot.d;
  AttnLayout lay = attn_workspace_layout(p, d, device_cu_count(p->rot_k->rot.device));
  tq_attn_params ps = *p;   // with the static scratch as the workspace (static_scratch)
  if (static_scratch) {
    if (lay.total > kAttnScratchBytes)
      return fail(TQ_ERR_WORKSPACE, std::string(who) + ": this call needs " + std::to_string(lay.total) +
                                        " bytes of scratch but the static scratch holds " +
                                        std::to_string(kAttnScratchBytes) +
                                        " (fewer num_splits, a smaller batch, or tq_attn_decode with a workspace)");
    if ((s = check_device(p->rot_k->rot, who))) return s;
    void* ptr = nullptr;
    hipError_t e = attn_scratch(p->rot_k->rot.device, &ptr);
    if (e != hipSuccess)
      return fail(TQ_ERR_HIP, std::string(who) + ": resolving the static scratch failed: " + hipGetErrorString(e));
    ps.workspace = ptr;
    ps.workspace_bytes = kAttnScratchBytes;
  } else {
    if (!p->workspace) return fail(TQ_ERR_WORKSPACE, std::string(who) + ": workspace is NULL");
    if (!aligned(p->workspace, 256)) return fail(TQ_ERR_ALIGN, std::string(who) + ": workspace must be 256-byte aligned");
    if (p->workspace_bytes < lay.total)
      return fail(TQ_ERR_WORKSPACE, std::string(who) + ": workspace_bytes = " + std::to_string(p->workspace_bytes) +
                                        " is smaller than the " + std::to_string(lay.total) + " bytes needed");
    if ((s = check_device(p->rot_k->rot, who))) return s;
  }
  const Codebook& cv = scores_only ? p->cb_k->cb : p->cb_v->cb;
  const Rotation& rv = scores_only ? p->rot_k->rot : p->rot_v->rot;
  return hip_status(launch_attention(&ps, p->cb_k->cb, cv, p->rot_k->rot, rv, scores, scores_only, lay,
                                     (hipStream_t)stream),
                    who);
}

int tq_scores_compressed(const tq_attn_params* p, float* scores, tq_stream_t stream) {
  return attn_common(p, scores, true, stream, "tq_scores_compressed");
}

int tq_attn_decode(const tq_attn_params* p, tq_stream_t stream) {
  return attn_common(p, nullptr, false, stream, "tq_attn_decode");
}

int tq_attn_decode_noalloc(const tq_attn_params* p, tq_stream_t stream) {
  return attn_common(p, nullptr, false, stream, "tq_attn_decode_noalloc", true);
}

}  // extern "C"

// ---- recent-token window append --------------------------------------------------------------

namespace {
struct WinLayout {
  size_t k_stage, v_stage, slot, total;
};
WinLayout win_layout(const tq_window_append_params* p, int d) {
  auto a256 = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t rows = (size_t)std::max(p->batch, 0) * std::max(p->num_kv_heads, 0) * std::max(p->n_new, 0);
  const size_t stage = a256(rows * d * dtype_size(p->window_dtype));
  WinLayout L;
  L.k_stage = 0;
  L.v_stage = stage;
  L.slot = 2 * stage;
  L.total = 2 * stage + a256(rows * sizeof(int64_t));
  if (L.total == 0) L.total = 256;
  return L;
}
}  // namespace

static int check_window(const tq_window_append_params* p, const char* who) {
  const std::string W(who);
  if (!p) return fail(TQ_ERR_NULL, W + ": params is NULL");
  int s = check_pair(p->cb_k, p->rot_k, who);
  if (s) return s;
  if ((s = check_pair(p->cb_v, p->rot_v, who))) return s;
  if (p->rot_v->rot.d != p->rot_k->rot.d) return fail(TQ_ERR_INVALID_ARG, W + ": K and V rotations have different d");
  if (p->rot_v->rot.device != p->rot_k->rot.device)
    return fail(TQ_ERR_NO_DEVICE, W + ": K and V rotations live on different devices");
  if (p->batch < 0 || p->num_kv_heads <= 0 || p->n_new < 0)
    return fail(TQ_ERR_INVALID_ARG, W + ": batch and n_new must be >= 0 and num_kv_heads > 0");
  if (p->window < 0) return fail(TQ_ERR_INVALID_ARG, W + ": window must be >= 0");
  if (!dtype_size(p->window_dtype))
    return fail(TQ_ERR_INVALID_ARG, W + ": window_dtype is not supported; accepted TQ_F32, TQ_BF16, TQ_F16");
  if (p->max_seq_len <= 0) return fail(TQ_ERR_INVALID_ARG, W + ": max_seq_len must be > 0");
  if (p->batch_per_rot < 0) return fail(TQ_ERR_INVALID_ARG, W + ": batch_per_rot must be >= 0");
  if (p->batch_per_rot > 0 && p->batch > 0) {
    int64_t need = ((int64_t)p->batch + p->batch_per_rot - 1) / p->batch_per_rot;
    if (need > p->rot_k->rot.n_rot || need > p->rot_v->rot.n_rot)
      return fail(TQ_ERR_INVALID_ARG, W + ": batch / batch_per_rot exceeds the rotation stack");
  }
  if (p->block_table) {
    if (p->block_size <= 0 || p->max_blocks_per_seq <= 0)
      return fail(TQ_ERR_INVALID_ARG, W + ": paged layout needs block_size > 0 and max_blocks_per_seq > 0");
    if ((int64_t)p->block_size * p->max_blocks_per_seq < p->max_seq_len)
      return fail(TQ_ERR_INVALID_ARG, W + ": block_size * max_blocks_per_seq < max_seq_len");
  }
  return TQ_OK;
}

size_t tq_window_append_workspace_size(const tq_window_append_params* p) {
  if (check_window(p, "tq_window_append_workspace_size")) return 0;
  return win_layout(p, p->rot_k->rot.d).total;
}

int tq_window_append(const tq_window_append_params* p, tq_stream_t stream) {
  const char* who = "tq_window_append";
  const std::string W(who);
  int s = check_window(p, who);
  if (s) return s;
  if (p->batch == 0 || p->n_new == 0) return TQ_OK;
  if (!p->k_new || !p->v_new) return fail(TQ_ERR_NULL, W + ": k_new / v_new is NULL");
  if (p->window > 0 && (!p->k_window || !p->v_window)) return fail(TQ_ERR_NULL, W + ": k_window / v_window is NULL");
  if (!p->seq_lens) return fail(TQ_ERR_NULL, W + ": seq_lens is NULL");
  if (!p->k_packed || !p->k_norms || !p->v_packed || !p->v_norms)
    return fail(TQ_ERR_NULL, W + ": the compressed cache pointers must not be NULL");
  if (!aligned(p->k_new, 16) || !aligned(p->v_new, 16) || !aligned(p->k_window, 16) || !aligned(p->v_window, 16))
    return fail(TQ_ERR_ALIGN, W + ": k_new, v_new, k_window and v_window must be 16-byte aligned");
  if (!aligned(p->k_packed, 8) || !aligned(p->v_packed, 8) || !aligned(p->k_norms, 4) || !aligned(p->v_norms, 4))
    return fail(TQ_ERR_ALIGN, W + ": packed caches must be 8-byte and norms 4-byte aligned");
  const int d = p->rot_k->rot.d;
  const WinLayout lay = win_layout(p, d);
  if (!p->workspace) return fail(TQ_ERR_WORKSPACE, W + ": workspace is NULL");
  if (!aligned(p->workspace, 256)) return fail(TQ_ERR_ALIGN, W + ": workspace must be 256-byte aligned");
  if (p->workspace_bytes < lay.total)
    return fail(TQ_ERR_WORKSPACE, W + ": workspace_bytes = " + std::to_string(p->workspace_bytes) + " < " +
                                      std::to_string(lay.total) + " needed");
  if ((s = check_device(p->rot_k->rot, who))) return s;
  WindowAppendLaunch L;
  const int64_t vpr = p->batch_per_rot > 0 ? (int64_t)p->num_kv_heads * p->n_new * p->batch_per_rot : 0;
  for (int side = 0; side < 2; ++side) {
    EncodeLaunch& e = side == 0 ? L.enc_k : L.enc_v;
    const tq_codebook_t* cb = side == 0 ? p->cb_k : p->cb_v;
    e.rot = side == 0 ? &p->rot_k->rot : &p->rot_v->rot;
    e.lv = make_levels(cb->cb);
    if (!lut_covers_unit_range(e.lv))
      return fail(TQ_ERR_INVALID_ARG, W + ": a codebook's boundaries are too close for the quantization table");
    e.bits = cb->cb.bits;
    e.x_dtype = p->window_dtype;
    e.vectors_per_rot = vpr;
    e.packed = side == 0 ? p->k_packed : p->v_packed;
    e.norms = side == 0 ? p->k_norms : p->v_norms;
    e.norm_correct = false;
  }
  uint8_t* ws = (uint8_t*)p->workspace;
  L.k_new = p->k_new;
  L.v_new = p->v_new;
  L.k_ring = p->k_window;
  L.v_ring = p->v_window;
  L.k_stage = ws + lay.k_stage;
  L.v_stage = ws + lay.v_stage;
  L.slot = (int64_t*)(ws + lay.slot);
  L.seq_lens = p->seq_lens;
  L.block_table = p->block_table;
  L.B = p->batch;
  L.Hkv = p->num_kv_heads;
  L.n_new = p->n_new;
  L.R = p->window;
  L.d = d;
  L.elem = dtype_size(p->window_dtype);
  L.max_seq_len = p->max_seq_len;
  L.block_size = p->block_table ? p->block_size : 1;
  L.mbps = p->max_blocks_per_seq;
  L.stream = (hipStream_t)stream;
  return hip_status(launch_window_append(L), who);
}

// ---- affine group quantization of values --------------------------------------------------------

static int gq_common(const char* who, int d, int bits, int64_t n) {
  const std::string W(who);
  if (d < 32 || d > 8192 || d % 32)
    return fail(TQ_ERR_INVALID_ARG, W + ": d = " + std::to_string(d) + " is not supported; accepted multiples of 32 in 32..8192");
  if (bits != 2 && bits != 3 && bits != 4 && bits != 8)
    return fail(TQ_ERR_INVALID_ARG, W + ": bits = " + std::to_string(bits) + " is not supported; accepted 2, 3, 4, 8");
  if (n < 0) return fail(TQ_ERR_INVALID_ARG, W + ": n must be >= 0");
  return TQ_OK;
}

int tq_gq_encode(int d, int bits, const void* x, int x_dtype, int64_t n, int64_t x_row_stride, uint8_t* packed,
                 uint16_t* scales, uint16_t* zeros, tq_stream_t stream) {
  const char* who = "tq_gq_encode";
  const std::string W(who);
  int s = gq_common(who, d, bits, n);
  if (s) return s;
  const int es = dtype_size(x_dtype);
  if (!es)
    return fail(TQ_ERR_INVALID_ARG, W + ": x_dtype = " + std::to_string(x_dtype) +
                                        " is not supported; accepted TQ_F32 (0), TQ_BF16 (1), TQ_F16 (2)");
  if (x_row_stride < d)
    return fail(TQ_ERR_INVALID_ARG, W + ": x_row_stride = " + std::to_string(x_row_stride) + " is smaller than d");
  if (n == 0) return TQ_OK;
  if (!x || !packed || !scales || !zeros) return fail(TQ_ERR_NULL, W + ": x, packed, scales and zeros must not be NULL");
  if (!aligned(x, 16) || (x_row_stride * es) % 16)
    return fail(TQ_ERR_ALIGN, W + ": x and x_row_stride * element size must be 16-byte aligned");
  if (!aligned(packed, 16) || !aligned(scales, 2) || !aligned(zeros, 2))
    return fail(TQ_ERR_ALIGN, W + ": packed must be 16-byte and scales / zeros 2-byte aligned");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(TQ_ERR_NO_DEVICE, W + ": no HIP device");
  GqLaunch L;
  L.encode = true;
  L.bits = bits;
  L.d = d;
  L.dtype = x_dtype;
  L.n = n;
  L.x_row_stride = x_row_stride;
  L.x = x;
  L.packed = packed;
  L.scales = scales;
  L.zeros = zeros;
  L.out = nullptr;
  L.stream = (hipStream_t)stream;
  return hip_status(launch_gq(L), who);
}

int tq_gq_decode(int d, int bits, const uint8_t* packed, const uint16_t* scales, const uint16_t* zeros, int64_t n,
                 void* out, int out_dtype, tq_stream_t stream) {
  const char* who = "tq_gq_decode";
  const std::string W(who);
  int s = gq_common(who, d, bits, n);
  if (s) return s;
  if (!dtype_size(out_dtype))
    return fail(TQ_ERR_INVALID_ARG, W + ": out_dtype = " + std::to_string(out_dtype) +
                                        " is not supported; accepted TQ_F32 (0), TQ_BF16 (1), TQ_F16 (2)");
  if (n == 0) return TQ_OK;
  if (!packed || !scales || !zeros || !out) return fail(TQ_ERR_NULL, W + ": packed, scales, zeros and out must not be NULL");
  if (!aligned(packed, 16) || !aligned(scales, 2) || !aligned(zeros, 2) || !aligned(out, 16))
    return fail(TQ_ERR_ALIGN, W + ": packed and out must be 16-byte and scales / zeros 2-byte aligned");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(TQ_ERR_NO_DEVICE, W + ": no HIP device");
  GqLaunch L;
  L.encode = false;
  L.bits = bits;
  L.d = d;
  L.dtype = out_dtype;
  L.n = n;
  L.x_row_stride = d;
  L.x = nullptr;
  L.packed = const_cast<uint8_t*>(packed);
  L.scales = const_cast<uint16_t*>(scales);
  L.zeros = const_cast<uint16_t*>(zeros);
  L.out = out;
  L.stream = (hipStream_t)stream;
  return hip_status(launch_gq(L), who);
}
