// Host side of libtq: codebook construction, rotation setup, context
// management and argument validation for every C-ABI entry point.
//
// Pages cited by title and section:
//  [ebisuda] "TurboQuant: Google's 6x KV Cache Compression Algorithm Gains
//            Open-Source Momentum", sections 第1段階 / 第2段階.
//  [gemilab] TurboQuant technical deep dive, section QJLの応用.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <string>
#include <thread>
#include <vector>

#include "tq_internal.h"

namespace tq {

static thread_local std::string g_last_error;

void set_error(const std::string &msg) { g_last_error = msg; }

tq_status fail(tq_status s, const std::string &msg) {
  g_last_error = msg;
  return s;
}

tq_status hip_fail(hipError_t e, const char *what) {
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return TQ_ERR_HIP;
}

int walsh_subset(int bits, int i) {
  int k = 0;
  for (int pc = 1; pc <= bits; pc += 2)
    for (int s = 1; s < (1 << bits); ++s)
      if (__builtin_popcount(s) == pc) {
        if (k == i) return s;
        ++k;
      }
  return 0;
}

// ---------------------------------------------------------------------------
// Coordinate law of a rotated unit vector ([ebisuda] 第1段階: Beta, close to
// N(0, 1/d)): f_d(x) = (1-x^2)^((d-3)/2) / B(1/2, (d-1)/2) on [-1, 1], i.e.
// (1+x)/2 ~ Beta(a, a) with a = (d-1)/2.
// ---------------------------------------------------------------------------

static double log_beta(double a, double b) { return std::lgamma(a) + std::lgamma(b) - std::lgamma(a + b); }

// Regularized incomplete beta I_x(a, b) from its continued fraction (DLMF
// 8.17.22), evaluated with the modified Lentz method; the reflection
// I_x(a,b) = 1 - I_{1-x}(b,a) keeps x below the convergence switch point.
static double inc_beta(double a, double b, double x) {
  if (x <= 0.0) return 0.0;
  if (x >= 1.0) return 1.0;
  if (x > (a + 1.0) / (a + b + 2.0)) return 1.0 - inc_beta(b, a, 1.0 - x);
  const double tiny = 1e-300;
  double f = 1.0, C = 1.0, D = 0.0;
  for (int j = 1; j < 20000; ++j) {
    double dj;
    if (j & 1) {
      int m = (j - 1) / 2;
      dj = -(a + m) * (a + b + m) * x / ((a + 2.0 * m) * (a + 2.0 * m + 1.0));
    } else {
      int m = j / 2;
      dj = m * (b - m) * x / ((a + 2.0 * m - 1.0) * (a + 2.0 * m));
    }
    D = 1.0 + dj * D;
    if (std::fabs(D) < tiny) D = tiny;
    C = 1.0 + dj / C;
    if (std::fabs(C) < tiny) C = tiny;
    D = 1.0 / D;
    double delta = C * D;
    f *= delta;
    if (std::fabs(delta - 1.0) < 1e-16) break;
  }
  double logpre = a * std::log(x) + b * std::log1p(-x) - log_beta(a, b);
  return std::exp(logpre) / (a * f);
}

static double coord_cdf(int d, double x) {
  if (x <= -1.0) return 0.0;
  if (x >= 1.0) return 1.0;
  double a = 0.5 * (d - 1);
  return inc_beta(a, a, 0.5 * (1.0 + x));
}

// (1 - x^2)^((d-1)/2) / B(1/2, (d-1)/2); antiderivative pieces of x f_d(x).
static double w_fun(int d, double x) {
  if (std::fabs(x) >= 1.0) return 0.0;
  return std::exp(0.5 * (d - 1) * std::log1p(-x * x) - log_beta(0.5, 0.5 * (d - 1)));
}

// Integral of x f_d over [a, b]: (w(a) - w(b)) / (d - 1).
static double first_moment(int d, double a, double b) { return (w_fun(d, a) - w_fun(d, b)) / (d - 1); }

// Integral of x^2 f_d over [a, b], integrating by parts once:
// [a w(a) - b w(b)]/(d-1) + B(1/2,(d+1)/2)/((d-1) B(1/2,(d-1)/2)) (F_{d+2}(b) - F_{d+2}(a)).
static double second_moment(int d, double a, double b) {
  double ratio = std::exp(log_beta(0.5, 0.5 * (d + 1)) - log_beta(0.5, 0.5 * (d - 1))) / (d - 1);
  return (a * w_fun(d, a) - b * w_fun(d, b)) / (d - 1) + ratio * (coord_cdf(d + 2, b) - coord_cdf(d + 2, a));
}

static double coord_quantile(int d, double p) {
  double lo = -1.0, hi = 1.0;
  for (int it = 0; it < 200; ++it) {
    double mid = 0.5 * (lo + hi);
    if (coord_cdf(d, mid) < p) lo = mid; else hi = mid;
  }
  return 0.5 * (lo + hi);
}

// Lloyd-Max ([ebisuda] 第1段階: continuous 1-D k-means minimizing MSE at a
// given bit width; precomputed per bit width, data-oblivious). Start from the
// centroids of 2^bits equal-mass cells, then alternate midpoint boundaries
// and conditional-mean centroids until no centroid moves by 1e-14; finally
// make the table exactly antisymmetric (f_d is even).
static std::vector<double> lloyd_max(int d, int bits) {
  const int L = 1 << bits;
  std::vector<double> e(L + 1), c(L);
  e[0] = -1.0;
  e[L] = 1.0;
  for (int i = 1; i < L; ++i) e[i] = coord_quantile(d, double(i) / L);
  for (int i = 0; i < L; ++i)
    c[i] = first_moment(d, e[i], e[i + 1]) / (coord_cdf(d, e[i + 1]) - coord_cdf(d, e[i]));
  for (int it = 0; it < 200000; ++it) {
    for (int i = 1; i < L; ++i) e[i] = 0.5 * (c[i - 1] + c[i]);
    double delta = 0.0;
    for (int i = 0; i < L; ++i) {
      double mass = coord_cdf(d, e[i + 1]) - coord_cdf(d, e[i]);
      double cn = first_moment(d, e[i], e[i + 1]) / mass;
      delta = std::max(delta, std::fabs(cn - c[i]));
      c[i] = cn;
    }
    if (delta < 1e-14) break;
  }
  std::vector<double> s(L);
  for (int i = 0; i < L; ++i) s[i] = 0.5 * (c[i] - c[L - 1 - i]);
  return s;
}

// ---------------------------------------------------------------------------
// Rotation: Householder QR of the caller's Gaussian matrix, fp64.
// ---------------------------------------------------------------------------

// Returns Pi = Q diag(sign(diag R)) (sign(0) = +1), row-major, as fp32.
static std::vector<float> rotation_from_gaussian(int n, const double *g) {
  std::vector<double> A((size_t)n * n), Q((size_t)n * n, 0.0);  // column-major
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j) A[(size_t)j * n + i] = g[(size_t)i * n + j];
  std::vector<std::vector<double>> V(n);
  std::vector<double> tau(n, 0.0), rdiag(n, 0.0);
  const unsigned hw = std::max(1u, std::min(8u, std::thread::hardware_concurrency()));

  auto apply = [&](double *M, int k, int j0, int j1) {  // columns [j0, j1) of M <- H_k M
    const double *v = V[k].data();
    const int len = n - k;
    for (int j = j0; j < j1; ++j) {
      double *col = M + (size_t)j * n + k;
      double s = 0.0;
      for (int i = 0; i < len; ++i) s += v[i] * col[i];
      s *= tau[k];
      for (int i = 0; i < len; ++i) col[i] -= s * v[i];
    }
  };
  auto parallel_apply = [&](double *M, int k, int j0, int j1) {
    int cols = j1 - j0;
    if (cols < 256 || hw == 1) {
      apply(M, k, j0, j1);
      return;
    }
    std::vector<std::thread> th;
    int per = (cols + hw - 1) / hw;
    for (unsigned t = 0; t < hw; ++t) {
      int a = j0 + (int)t * per, b = std::min(j1, a + per);
      if (a < b) th.emplace_back(apply, M, k, a, b);
    }
    for (auto &t : th) t.join();
  };

  for (int k = 0; k < n; ++k) {
    double *x = A.data() + (size_t)k * n + k;
    const int len = n - k;
    double nrm2 = 0.0;
    for (int i = 0; i < len; ++i) nrm2 += x[i] * x[i];
    double nrm = std::sqrt(nrm2);
    double alpha = (x[0] > 0.0) ? -nrm : nrm;  // R_kk; v = x - alpha e1 avoids cancellation
    V[k].assign(x, x + len);
    V[k][0] -= alpha;
    double vn2 = 0.0;
    for (int i = 0; i < len; ++i) vn2 += V[k][i] * V[k][i];
    tau[k] = vn2 > 0.0 ? 2.0 / vn2 : 0.0;
    rdiag[k] = alpha;
    if (k + 1 < n) parallel_apply(A.data(), k, k + 1, n);
  }
  for (int i = 0; i < n; ++i) Q[(size_t)i * n + i] = 1.0;
  for (int k = n - 1; k >= 0; --k) parallel_apply(Q.data(), k, k, n);
  std::vector<float> pi((size_t)n * n);
  for (int j = 0; j < n; ++j) {
    double sgn = rdiag[j] < 0.0 ? -1.0 : 1.0;
    for (int i = 0; i < n; ++i) pi[(size_t)i * n + j] = (float)(sgn * Q[(size_t)j * n + i]);
  }
  return pi;
}

// ---------------------------------------------------------------------------
// Seeded Gaussian draws for the rotation's and the sketch's matrices: a
// counter-based generator (the SplitMix64 output function of Steele, Lea &
// Flood, OOPSLA 2014, applied to seed ^ stream * GAMMA ^ counter) and the
// Box-Muller transform (Box & Muller 1958), fp64, filled row-major.
// ---------------------------------------------------------------------------

static inline uint64_t splitmix64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// n (even) N(0,1) values: entry 2k = r cos(2 pi u_{2k+1}), 2k + 1 = r sin(2 pi u_{2k+1}),
// r = sqrt(-2 ln(1 - u_{2k})), u_i = (mix(key ^ i) >> 11) 2^-53, key = seed ^ stream * GAMMA
static void seeded_gaussian(uint64_t seed, uint64_t stream, int64_t n, double *out) {
  const uint64_t key = seed ^ (stream * 0x9E3779B97F4A7C15ull);
  for (int64_t k = 0; 2 * k + 1 < n; ++k) {
    const double u1 = (double)(splitmix64_mix(key ^ (uint64_t)(2 * k)) >> 11) * 0x1p-53;
    const double u2 = (double)(splitmix64_mix(key ^ (uint64_t)(2 * k + 1)) >> 11) * 0x1p-53;
    const double r = std::sqrt(-2.0 * std::log(1.0 - u1));  // 1 - u1 is exact
    const double a = 2.0 * M_PI * u2;
    out[2 * k] = r * std::cos(a);
    out[2 * k + 1] = r * std::sin(a);
  }
}

}  // namespace tq

using namespace tq;

extern "C" {

const char *tq_last_error(void) { return g_last_error.c_str(); }

int32_t tq_format_version(void) { return TQ_FORMAT_VERSION; }

tq_status tq_read_probe(const void *d_src, size_t bytes, int32_t grid, uint32_t *d_sink, void *stream) {
  if (!d_src || !d_sink) return fail(TQ_ERR_ARG, "tq_read_probe: NULL buffer");
  if (((uintptr_t)d_src & 15) != 0 || (bytes & 15) != 0 || bytes == 0)
    return fail(TQ_ERR_ARG, "tq_read_probe: source must be 16-byte aligned and a positive multiple of 16 bytes");
  if (grid < 1 || grid > 65536) return fail(TQ_ERR_ARG, "tq_read_probe: grid must be in [1, 65536]");
  hipError_t e = launch_read_probe(d_src, bytes, grid, d_sink, (hipStream_t)stream);
  return e == hipSuccess ? TQ_OK : hip_fail(e, "tq_read_probe");
}

// events armed by tq_time_next_decode on this thread (both NULL when disarmed)
static thread_local hipEvent_t g_decode_ev[2] = {nullptr, nullptr};

tq_status tq_time_next_decode(void *start_event, void *stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr))
    return fail(TQ_ERR_ARG, "tq_time_next_decode: pass both events or neither");
  g_decode_ev[0] = (hipEvent_t)start_event;
  g_decode_ev[1] = (hipEvent_t)stop_event;
  return TQ_OK;
}

// takes the armed events (if any) and disarms the thread
static void take_decode_events(hipEvent_t ev[2]) {
  ev[0] = g_decode_ev[0];
  ev[1] = g_decode_ev[1];
  g_decode_ev[0] = g_decode_ev[1] = nullptr;
}

tq_status tq_codebook_build(int32_t d, int32_t bits, tq_codebook *out) {
  if (!out) return fail(TQ_ERR_ARG, "tq_codebook_build: out is NULL");
  if (d < 3 || d > TQ_MAX_DIM) return fail(TQ_ERR_UNSUPPORTED, "tq_codebook_build: d must be in [3, 4096]");
  if (bits < 1 || bits > TQ_MAX_BITS) return fail(TQ_ERR_UNSUPPORTED, "tq_codebook_build: bits must be in [1, 4]");
  const int L = 1 << bits;
  std::vector<double> c = lloyd_max(d, bits);
  tq_codebook cb;
  std::memset(&cb, 0, sizeof(cb));
  cb.d = d;
  cb.bits = bits;
  for (int i = 0; i < L; ++i) cb.centroid[i] = (float)c[i];
  for (int i = 0; i + 1 < L; ++i) cb.boundary[i] = (float)(0.5 * (c[i] + c[i + 1]));
  // Odd Walsh coefficients of the stored table: c[idx] = sum_S w_S prod_{p in S}(2 b_p - 1).
  for (int i = 0; i < (L >> 1); ++i) {
    int S = walsh_subset(bits, i);
    double acc = 0.0;
    for (int idx = 0; idx < L; ++idx) {
      int par = __builtin_popcount(~idx & S) & 1;  // number of zero bits in S
      acc += (par ? -1.0 : 1.0) * (double)cb.centroid[idx];
    }
    cb.walsh[i] = (float)(acc / L);
  }
  // Analytic per-coordinate MSE of the stored tables.
  double D = 0.0;
  for (int i = 0; i < L; ++i) {
    double a = i == 0 ? -1.0 : (double)cb.boundary[i - 1];
    double b = i == L - 1 ? 1.0 : (double)cb.boundary[i];
    double ci = cb.centroid[i];
    double m0 = coord_cdf(d, b) - coord_cdf(d, a);
    D += second_moment(d, a, b) - 2.0 * ci * first_moment(d, a, b) + ci * ci * m0;
  }
  cb.distortion = D;
  *out = cb;
  return TQ_OK;
}

// ---------------------------------------------------------------------------
// PolarQuant angle codebooks. Angle of level l >= 2 of a random direction,
// m = 2^(l-1): sin^2(psi) ~ Beta(m/2, m/2), density
// 2^(2-m) sin^(m-1)(2 psi) / B(m/2, m/2) on [0, pi/2]; level 1 uniform on the
// circle (cells from -pi). Lloyd-Max per level, symmetric about pi/4.
// ---------------------------------------------------------------------------

static double angle_pdf(int m, double psi) {
  const double s = std::sin(2.0 * psi);
  if (s <= 0.0) return m == 1 ? std::exp((2 - m) * std::log(2.0) - log_beta(0.5 * m, 0.5 * m)) : 0.0;
  return std::exp((2 - m) * std::log(2.0) - log_beta(0.5 * m, 0.5 * m) + (m - 1) * std::log(s));
}

static double angle_cdf(int m, double psi) {
  const double p = std::min(std::max(psi, 0.0), M_PI / 2);
  const double u = std::sin(p);
  return inc_beta(0.5 * m, 0.5 * m, u * u);
}

// int_a^b psi f(psi) dpsi: composite 16-point Gauss-Legendre on 32 panels
static double angle_moment1(int m, double a, double b) {
  static const double x[8] = {0.0950125098376374, 0.2816035507792589, 0.4580167776572274, 0.6178762444026438,
                              0.7554044083550030, 0.8656312023878318, 0.9445750230732326, 0.9894009349916499};
  static const double w[8] = {0.1894506104550685, 0.1826034150449236, 0.1691565193950025, 0.1495959888165767,
                              0.1246289712555339, 0.0951585116824928, 0.0622535239386479, 0.0271524594117541};
  const int P = 32;
  const double h = (b - a) / P;
  double acc = 0.0;
  for (int k = 0; k < P; ++k) {
    const double c = a + (k + 0.5) * h, r = 0.5 * h;
    for (int i = 0; i < 8; ++i) {
      const double t1 = c - r * x[i], t2 = c + r * x[i];
      acc += w[i] * r * (t1 * angle_pdf(m, t1) + t2 * angle_pdf(m, t2));
    }
  }
  return acc;
}

static std::vector<double> lloyd_max_angle(int level, int bits) {
  const int L = 1 << bits;
  std::vector<double> c(L);
  if (level == 1) {
    for (int i = 0; i < L; ++i) c[i] = -M_PI + (i + 0.5) * (2.0 * M_PI / L);
    return c;
  }
  const int m = 1 << (level - 1);
  std::vector<double> e(L + 1);
  e[0] = 0.0;
  e[L] = M_PI / 2;
  for (int i = 1; i < L; ++i) {  // equal-mass start: bisection on the CDF
    double lo = 0.0, hi = M_PI / 2;
    for (int it = 0; it < 200; ++it) {
      const double mid = 0.5 * (lo + hi);
      if (angle_cdf(m, mid) < double(i) / L) lo = mid; else hi = mid;
    }
    e[i] = 0.5 * (lo + hi);
  }
  auto centroids = [&]() {
    for (int i = 0; i < L; ++i) c[i] = angle_moment1(m, e[i], e[i + 1]) / (angle_cdf(m, e[i + 1]) - angle_cdf(m, e[i]));
  };
  centroids();
  for (int it = 0; it < 10000; ++it) {
    for (int i = 1; i < L; ++i) e[i] = 0.5 * (c[i - 1] + c[i]);
    std::vector<double> old = c;
    centroids();
    double delta = 0.0;
    for (int i = 0; i < L; ++i) delta = std::max(delta, std::fabs(c[i] - old[i]));
    if (delta < 1e-12) break;
  }
  std::vector<double> s(L);
  for (int i = 0; i < L; ++i) s[i] = 0.5 * (c[i] + (M_PI / 2 - c[L - 1 - i]));
  return s;
}

tq_status tq_angle_codebook_build(int32_t level, int32_t bits, tq_angle_codebook *out) {
  if (!out) return fail(TQ_ERR_ARG, "tq_angle_codebook_build: out is NULL");
  if (level < 1 || level > TQ_POLAR_MAX_LEVEL)
    return fail(TQ_ERR_UNSUPPORTED, "tq_angle_codebook_build: level must be in [1, 12]");
  if (bits < 1 || bits > TQ_MAX_BITS) return fail(TQ_ERR_UNSUPPORTED, "tq_angle_codebook_build: bits must be in [1, 4]");
  const int L = 1 << bits;
  std::vector<double> c = lloyd_max_angle(level, bits);
  tq_angle_codebook cb;
  std::memset(&cb, 0, sizeof(cb));
  cb.level = level;
  cb.bits = bits;
  for (int i = 0; i < L; ++i) {
    cb.centroid[i] = c[i];
    cb.cos_c[i] = (float)std::cos(c[i]);
    cb.sin_c[i] = (float)std::sin(c[i]);
  }
  for (int i = 0; i + 1 < L; ++i)
    cb.boundary[i] = (float)(level == 1 ? -M_PI + (i + 1) * (2.0 * M_PI / L) : 0.5 * (c[i] + c[i + 1]));
  *out = cb;
  return TQ_OK;
}

tq_status tq_rotation_build(int32_t d, const double *h_g, float *h_out) {
  if (!h_g || !h_out) return fail(TQ_ERR_ARG, "tq_rotation_build: NULL argument");
  if (d < 2 || d > TQ_MAX_DIM) return fail(TQ_ERR_UNSUPPORTED, "tq_rotation_build: d must be in [2, 4096]");
  std::vector<float> pi = rotation_from_gaussian(d, h_g);
  std::memcpy(h_out, pi.data(), pi.size() * sizeof(float));
  return TQ_OK;
}

// bf16 with round-to-nearest-even of a finite fp32 value, and back
static uint16_t bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
static float bf16_value(uint16_t h) {
  const uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

tq_status tq_ctx_create(int32_t d, const double *h_g_rot, const double *h_g_sketch, tq_ctx **out) {
  if (!out || !h_g_rot || !h_g_sketch) return fail(TQ_ERR_ARG, "tq_ctx_create: NULL argument");
  *out = nullptr;
  if (d < 32 || d > TQ_MAX_DIM || (d % 32) != 0)
    return fail(TQ_ERR_UNSUPPORTED, "tq_ctx_create: d must be a multiple of 32 in [32, 4096]");
  tq_ctx *ctx = new (std::nothrow) tq_ctx();
  if (!ctx) return fail(TQ_ERR_NOMEM, "tq_ctx_create: host allocation failed");
  ctx->d = d;
  hipError_t e = hipGetDevice(&ctx->device);
  if (e != hipSuccess) {
    delete ctx;
    return hip_fail(e, "tq_ctx_create: hipGetDevice");
  }
  // the device address of this device's scratch array (tq_attention_decode_noalloc)
  if ((e = scratch_init(ctx->device)) != hipSuccess) {
    delete ctx;
    return hip_fail(e, "tq_ctx_create: scratch symbol address");
  }
  ctx->rot = rotation_from_gaussian(d, h_g_rot);
  ctx->sketch.resize((size_t)d * d);
  for (size_t i = 0; i < (size_t)d * d; ++i) ctx->sketch[i] = (float)h_g_sketch[i];
  std::memset(&ctx->h_tables, 0, sizeof(ctx->h_tables));
  for (int b = 1; b <= TQ_MAX_BITS; ++b) {
    tq_status s = tq_codebook_build(d, b, &ctx->cb[b]);
    if (s != TQ_OK) {
      delete ctx;
      return s;
    }
    const int L = 1 << b;
    for (int i = 0; i < L; ++i) ctx->h_tables.centroid[b][i] = ctx->cb[b].centroid[i];
    for (int i = 0; i + 1 < L; ++i) ctx->h_tables.boundary[b][i] = ctx->cb[b].boundary[i];
    for (int i = L - 1; i < 16; ++i) ctx->h_tables.boundary[b][i] = INFINITY;
    for (int i = 0; i < (L >> 1); ++i) ctx->h_tables.walsh[b][i] = ctx->cb[b].walsh[i];
    ctx->h_tables.ctop[b] = ctx->cb[b].centroid[L - 1];
  }
  // PolarQuant angle tables (the GPU polar path supports d = 128: levels 1..7)
  if (d == 128) {
    for (int lv = 1; lv <= 7; ++lv)
      for (int b = 1; b <= TQ_MAX_BITS; ++b) {
        tq_angle_codebook acb;
        tq_status s = tq_angle_codebook_build(lv, b, &acb);
        if (s != TQ_OK) {
          delete ctx;
          return s;
        }
        const int L = 1 << b;
        for (int i = 0; i < 16; ++i) ctx->h_tables.pbound[lv][b][i] = i + 1 < L ? acb.boundary[i] : INFINITY;
        for (int i = 0; i < L; ++i) {
          ctx->h_tables.pcos[lv][b][i] = acb.cos_c[i];
          ctx->h_tables.psin[lv][b][i] = acb.sin_c[i];
        }
      }
  }
  const size_t mat = (size_t)d * d * sizeof(float);
  if ((e = hipMalloc(&ctx->d_rot, mat)) != hipSuccess || (e = hipMalloc(&ctx->d_sketch, mat)) != hipSuccess ||
      (e = hipMalloc(&ctx->d_rot_t, mat)) != hipSuccess || (e = hipMalloc(&ctx->d_sketch_t, mat)) != hipSuccess ||
      (e = hipMalloc(&ctx->d_rs_t, 2 * mat)) != hipSuccess ||
      (e = hipMalloc(&ctx->d_tables, sizeof(DeviceTables))) != hipSuccess) {
    tq_ctx_destroy(ctx);
    return fail(TQ_ERR_NOMEM, std::string("tq_ctx_create: hipMalloc: ") + hipGetErrorString(e));
  }
  std::vector<float> rt((size_t)d * d), st((size_t)d * d), rst((size_t)2 * d * d);
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) {
      rt[(size_t)j * d + i] = ctx->rot[(size_t)i * d + j];
      st[(size_t)j * d + i] = ctx->sketch[(size_t)i * d + j];
    }
  // S Pi in fp64 from the fp32 tables, rounded to fp32; stored with Pi as [Pi ; S Pi]^T
  // (only the d = 128 decode path reads it)
  for (int i = 0; i < (d == 128 ? d : 0); ++i) {
    std::vector<double> row(d, 0.0);
    for (int k = 0; k < d; ++k) {
      const double sik = ctx->sketch[(size_t)i * d + k];
      for (int j = 0; j < d; ++j) row[j] += sik * (double)ctx->rot[(size_t)k * d + j];
    }
    for (int j = 0; j < d; ++j) {
      rst[(size_t)j * 2 * d + i] = ctx->rot[(size_t)i * d + j];
      rst[(size_t)j * 2 * d + d + i] = (float)row[j];
    }
  }
  // d = 128: Pi as three bf16 parts and S as two, for the bf16-MFMA quantizer
  if (d == 128) {
    std::vector<uint16_t> r3((size_t)3 * d * d), s2((size_t)2 * d * d);
    for (size_t i = 0; i < (size_t)d * d; ++i) {
      float rem = ctx->rot[i];
      for (int p = 0; p < 3; ++p) {
        r3[(size_t)p * d * d + i] = bf16_rne(rem);
        rem -= bf16_value(r3[(size_t)p * d * d + i]);
      }
      rem = ctx->sketch[i];
      for (int p = 0; p < 2; ++p) {
        s2[(size_t)p * d * d + i] = bf16_rne(rem);
        rem -= bf16_value(s2[(size_t)p * d * d + i]);
      }
    }
    if ((e = hipMalloc(&ctx->d_rot3, r3.size() * 2)) != hipSuccess ||
        (e = hipMalloc(&ctx->d_sk2, s2.size() * 2)) != hipSuccess ||
        (e = hipMemcpy(ctx->d_rot3, r3.data(), r3.size() * 2, hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipMemcpy(ctx->d_sk2, s2.data(), s2.size() * 2, hipMemcpyHostToDevice)) != hipSuccess) {
      tq_ctx_destroy(ctx);
      return hip_fail(e, "tq_ctx_create: bf16 parts");
    }
  }
  if ((e = hipMemcpy(ctx->d_rot, ctx->rot.data(), mat, hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipMemcpy(ctx->d_rot_t, rt.data(), mat, hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipMemcpy(ctx->d_sketch_t, st.data(), mat, hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipMemcpy(ctx->d_rs_t, rst.data(), 2 * mat, hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipMemcpy(ctx->d_sketch, ctx->sketch.data(), mat, hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipMemcpy(ctx->d_tables, &ctx->h_tables, sizeof(DeviceTables), hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipDeviceSynchronize()) != hipSuccess) {
    tq_ctx_destroy(ctx);
    return hip_fail(e, "tq_ctx_create: upload");
  }
  *out = ctx;
  return TQ_OK;
}

tq_status tq_gaussian_matrix(uint64_t seed, uint32_t stream, int32_t rows, int32_t cols, double *h_out) {
  if (!h_out) return fail(TQ_ERR_ARG, "tq_gaussian_matrix: h_out is NULL");
  if (rows <= 0 || cols <= 0 || (((int64_t)rows * cols) & 1) != 0)
    return fail(TQ_ERR_ARG, "tq_gaussian_matrix: rows and cols must be positive with an even product");
  seeded_gaussian(seed, stream, (int64_t)rows * cols, h_out);
  return TQ_OK;
}

tq_status tq_ctx_create_seeded(int32_t d, uint64_t seed, tq_ctx **out) {
  if (!out) return fail(TQ_ERR_ARG, "tq_ctx_create_seeded: out is NULL");
  *out = nullptr;
  if (d < 32 || d > TQ_MAX_DIM || (d % 32) != 0)
    return fail(TQ_ERR_UNSUPPORTED, "tq_ctx_create_seeded: d must be a multiple of 32 in [32, 4096]");
  std::vector<double> g_rot, g_sk;
  try {
    g_rot.resize((size_t)d * d);
    g_sk.resize((size_t)d * d);
  } catch (...) {
    return fail(TQ_ERR_NOMEM, "tq_ctx_create_seeded: host allocation failed");
  }
  seeded_gaussian(seed, TQ_STREAM_ROTATION, (int64_t)d * d, g_rot.data());
  seeded_gaussian(seed, TQ_STREAM_SKETCH, (int64_t)d * d, g_sk.data());
  return tq_ctx_create(d, g_rot.data(), g_sk.data(), out);
}

tq_status tq_ctx_destroy(tq_ctx *ctx) {
  if (!ctx) return fail(TQ_ERR_ARG, "tq_ctx_destroy: NULL ctx");
  (void)hipDeviceSynchronize();
  if (ctx->d_rot) (void)hipFree(ctx->d_rot);
  if (ctx->d_sketch) (void)hipFree(ctx->d_sketch);
  if (ctx->d_tables) (void)hipFree(ctx->d_tables);
  if (ctx->d_rot_t) (void)hipFree(ctx->d_rot_t);
  if (ctx->d_sketch_t) (void)hipFree(ctx->d_sketch_t);
  if (ctx->d_rs_t) (void)hipFree(ctx->d_rs_t);
  if (ctx->d_rot3) (void)hipFree(ctx->d_rot3);
  if (ctx->d_sk2) (void)hipFree(ctx->d_sk2);
  delete ctx;
  return TQ_OK;
}

int32_t tq_ctx_dim(const tq_ctx *ctx) { return ctx ? ctx->d : 0; }

tq_status tq_ctx_export(const tq_ctx *ctx, float *h_rot, float *h_sketch) {
  if (!ctx) return fail(TQ_ERR_ARG, "tq_ctx_export: NULL ctx");
  if (h_rot) std::memcpy(h_rot, ctx->rot.data(), ctx->rot.size() * sizeof(float));
  if (h_sketch) std::memcpy(h_sketch, ctx->sketch.data(), ctx->sketch.size() * sizeof(float));
  return TQ_OK;
}

tq_status tq_ctx_codebook(const tq_ctx *ctx, int32_t bits, tq_codebook *out) {
  if (!ctx || !out) return fail(TQ_ERR_ARG, "tq_ctx_codebook: NULL argument");
  if (bits < 1 || bits > TQ_MAX_BITS) return fail(TQ_ERR_UNSUPPORTED, "tq_ctx_codebook: bits must be in [1, 4]");
  *out = ctx->cb[bits];
  return TQ_OK;
}

// ---------------------------------------------------------------------------
// Hot-path entry points: validation, then one asynchronous launch sequence.
// ---------------------------------------------------------------------------

static tq_status check_device(const tq_ctx *ctx, const char *fn) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, fn);
  if (dev != ctx->device) return fail(TQ_ERR_ARG, std::string(fn) + ": current device differs from the context's");
  return TQ_OK;
}

static tq_status check_packed(const tq_ctx *ctx, const tq_packed *p, int want_key, const char *fn) {
  if (!p || !p->bits || !p->norms) return fail(TQ_ERR_ARG, std::string(fn) + ": packed array or its pointers NULL");
  if ((p->is_key != 0) != (want_key != 0))
    return fail(TQ_ERR_ARG, std::string(fn) + (want_key ? ": expected a key array" : ": expected a value array"));
  if (p->qjl != 0 && p->qjl != 1) return fail(TQ_ERR_ARG, std::string(fn) + ": qjl must be 0 or 1");
  if (p->norm_f16 != 0 && p->norm_f16 != 1) return fail(TQ_ERR_ARG, std::string(fn) + ": norm_f16 must be 0 or 1");
  if (!p->is_key && p->qjl) return fail(TQ_ERR_ARG, std::string(fn) + ": value arrays have no QJL stage (qjl = 0)");
  if (p->mse_bits < (p->is_key && p->qjl ? 0 : 1) || p->mse_bits > TQ_MAX_BITS)
    return fail(TQ_ERR_UNSUPPORTED, std::string(fn) + ": mse_bits must be in [1, 4] ([0, 4] for keys with qjl = 1)");
  if (p->n < 0) return fail(TQ_ERR_ARG, std::string(fn) + ": negative record count");
  if (!p->is_key && (p->n % 32) != 0) return fail(TQ_ERR_ARG, std::string(fn) + ": value capacity must be a multiple of 32");
  (void)ctx;
  return TQ_OK;
}

size_t tq_quantize_ws_bytes(const tq_ctx *ctx, int64_t n_streams, int64_t n_tokens, int32_t is_key) {
  if (!ctx || !is_key || n_streams <= 0 || n_tokens <= 0) return 0;
  return (size_t)n_streams * (size_t)n_tokens * (size_t)ctx->d * sizeof(float);
}

tq_status tq_quantize_kv(const tq_ctx *ctx, const void *d_x, tq_dtype dtype, int64_t n_streams, int64_t n_tokens,
                         int64_t x_stream_stride, int64_t x_token_stride, const tq_packed *out,
                         int64_t out_stream_stride, int64_t out_offset, void *d_work, size_t work_bytes,
                         void *stream) {
  const char *fn = "tq_quantize_kv";
  if (!ctx) return fail(TQ_ERR_ARG, "tq_quantize_kv: NULL ctx");
  if (!out) return fail(TQ_ERR_ARG, "tq_quantize_kv: NULL out");
  tq_status s = check_packed(ctx, out, out->is_key, fn);
  if (s != TQ_OK) return s;
  if (dtype != TQ_F32 && dtype != TQ_BF16) return fail(TQ_ERR_ARG, "tq_quantize_kv: dtype must be TQ_F32 or TQ_BF16");
  if (n_streams < 0 || n_tokens < 0 || out_offset < 0 || out_stream_stride < 0 || x_stream_stride < 0 ||
      x_token_stride < 0)
    return fail(TQ_ERR_ARG, "tq_quantize_kv: negative size, stride or offset");
  if (n_streams == 0 || n_tokens == 0) return TQ_OK;
  if (!d_x) return fail(TQ_ERR_ARG, "tq_quantize_kv: NULL input");
  if (x_token_stride < ctx->d && n_tokens > 1) return fail(TQ_ERR_ARG, "tq_quantize_kv: token stride < d");
  if ((x_token_stride % 8) != 0 || (x_stream_stride % 8) != 0 || ((uintptr_t)d_x % 16) != 0)
    return fail(TQ_ERR_ARG, "tq_quantize_kv: input must be 16-byte aligned with strides that are multiples of 8");
  if (n_streams > 65535) return fail(TQ_ERR_UNSUPPORTED, "tq_quantize_kv: at most 65535 streams per call");
  if (n_streams > 1 && out_stream_stride < out_offset + n_tokens)
    return fail(TQ_ERR_ARG, "tq_quantize_kv: output streams overlap (out_stream_stride < out_offset + n_tokens)");
  int64_t last = (n_streams - 1) * out_stream_stride + out_offset + n_tokens;
  if (last > out->n) return fail(TQ_ERR_ARG, "tq_quantize_kv: records past the end of the output array");
  if (!out->is_key && ((out_offset % 32) != 0 || (out_stream_stride % 32) != 0))
    return fail(TQ_ERR_ARG, "tq_quantize_kv: value offsets and stream strides must be multiples of 32");
  if (out->is_key) {
    size_t need = tq_quantize_ws_bytes(ctx, n_streams, n_tokens, 1);
    if (!d_work || work_bytes < need)
      return fail(TQ_ERR_CAPACITY, "tq_quantize_kv: key workspace smaller than tq_quantize_ws_bytes()");
  }
  if ((s = check_device(ctx, fn)) != TQ_OK) return s;
  RecMap map;
  map.os = out_stream_stride;
  map.oo = out_offset;
  hipError_t e;
  if (out->is_key)
    e = launch_quantize_keys(ctx, d_x, dtype == TQ_BF16, n_streams, n_tokens, x_stream_stride, x_token_stride, out,
                             map, (float *)d_work, (hipStream_t)stream);
  else
    e = launch_quantize_values(ctx, d_x, dtype == TQ_BF16, n_streams, n_tokens, x_stream_stride, x_token_stride,
                               out, map, (hipStream_t)stream);
  return e == hipSuccess ? TQ_OK : hip_fail(e, fn);
}

static tq_status check_cache(const tq_ctx *ctx, const tq_kv_cache *c, const char *fn) {
  if (!c) return fail(TQ_ERR_ARG, std::string(fn) + ": NULL cache");
  tq_status s = check_packed(ctx, &c->k, 1, fn);
  if (s == TQ_OK) s = check_packed(ctx, &c->v, 0, fn);
  if (s != TQ_OK) return s;
  if (c->k.norm_f16 != c->v.norm_f16)
    return fail(TQ_ERR_ARG, std::string(fn) + ": keys and values of a cache must store their norms alike (norm_f16)");
  if (c->batch <= 0 || c->kv_heads <= 0 || c->capacity <= 0 || (c->capacity % 32) != 0)
    return fail(TQ_ERR_ARG, std::string(fn) + ": batch, kv_heads > 0 and capacity a positive multiple of 32 required");
  if (c->d_block_table == nullptr) {
    int64_t recs = (int64_t)c->batch * c->kv_heads * c->capacity;
    if (c->k.n < recs || c->v.n < recs)
      return fail(TQ_ERR_ARG, std::string(fn) + ": record arrays smaller than batch*kv_heads*capacity");
  } else {
    if (c->page_tokens <= 0 || (c->page_tokens % 256) != 0 || (c->capacity % c->page_tokens) != 0)
      return fail(TQ_ERR_ARG, std::string(fn) + ": page_tokens must be a positive multiple of 256 dividing capacity");
    const int64_t page_recs = (int64_t)c->kv_heads * c->page_tokens;
    if (c->k.n != c->v.n || c->k.n < page_recs || (c->k.n % page_recs) != 0 || c->k.n / page_recs > INT32_MAX)
      return fail(TQ_ERR_ARG, std::string(fn) + ": paged record arrays must hold the same whole number of pages");
  }
  if (!c->d_seq_len) return fail(TQ_ERR_ARG, std::string(fn) + ": NULL d_seq_len");
  if (c->host_max_len < 0 || c->host_max_len > c->capacity)
    return fail(TQ_ERR_ARG, std::string(fn) + ": host_max_len outside [0, capacity]");
  return TQ_OK;
}

tq_status tq_cache_write(const tq_ctx *ctx, const tq_kv_cache *cache, const void *d_k, const void *d_v,
                         tq_dtype dtype, int64_t n_tokens, int64_t x_stream_stride, int64_t x_token_stride,
                         int64_t pos0, void *d_work, size_t work_bytes, void *stream) {
  const char *fn = "tq_cache_write";
  if (!ctx) return fail(TQ_ERR_ARG, "tq_cache_write: NULL ctx");
  tq_status s = check_cache(ctx, cache, fn);
  if (s != TQ_OK) return s;
  if (dtype != TQ_F32 && dtype != TQ_BF16) return fail(TQ_ERR_ARG, "tq_cache_write: dtype must be TQ_F32 or TQ_BF16");
  if (n_tokens < 0 || pos0 < 0 || x_stream_stride < 0 || x_token_stride < 0)
    return fail(TQ_ERR_ARG, "tq_cache_write: negative size, stride or position");
  if ((pos0 % 32) != 0) return fail(TQ_ERR_ARG, "tq_cache_write: pos0 must be a multiple of 32");
  if (pos0 + n_tokens > cache->capacity) return fail(TQ_ERR_ARG, "tq_cache_write: positions past capacity");
  if (n_tokens == 0) return TQ_OK;
  if (!d_k || !d_v) return fail(TQ_ERR_ARG, "tq_cache_write: NULL input");
  if (x_token_stride < ctx->d && n_tokens > 1) return fail(TQ_ERR_ARG, "tq_cache_write: token stride < d");
  if ((x_token_stride % 8) != 0 || (x_stream_stride % 8) != 0 || ((uintptr_t)d_k % 16) != 0 || ((uintptr_t)d_v % 16) != 0)
    return fail(TQ_ERR_ARG, "tq_cache_write: inputs must be 16-byte aligned with strides that are multiples of 8");
  const int64_t n_streams = (int64_t)cache->batch * cache->kv_heads;
  if (n_streams > 65535) return fail(TQ_ERR_UNSUPPORTED, "tq_cache_write: at most 65535 streams");
  size_t need = tq_quantize_ws_bytes(ctx, n_streams, n_tokens, 1);
  if (!d_work || work_bytes < need) return fail(TQ_ERR_CAPACITY, "tq_cache_write: workspace smaller than tq_quantize_ws_bytes()");
  if ((s = check_device(ctx, fn)) != TQ_OK) return s;
  const RecMap map = cache_map(cache, pos0);
  hipError_t e = launch_quantize_keys(ctx, d_k, dtype == TQ_BF16, n_streams, n_tokens, x_stream_stride, x_token_stride,
                                      &cache->k, map, (float *)d_work, (hipStream_t)stream);
  if (e == hipSuccess)
    e = launch_quantize_values(ctx, d_v, dtype == TQ_BF16, n_streams, n_tokens, x_stream_stride, x_token_stride,
                               &cache->v, map, (hipStream_t)stream);
  return e == hipSuccess ? TQ_OK : hip_fail(e, fn);
}

tq_status tq_append_token(const tq_ctx *ctx, tq_kv_cache *cache, const void *d_k, const void *d_v, tq_dtype dtype,
                          void *stream) {
  const char *fn = "tq_append_token";
  if (!ctx) return fail(TQ_ERR_ARG, "tq_append_token: NULL ctx");
  tq_status s = check_cache(ctx, cache, fn);
  if (s != TQ_OK) return s;
  if (!d_k || !d_v) return fail(TQ_ERR_ARG, "tq_append_token: NULL input");
  if (dtype != TQ_F32 && dtype != TQ_BF16) return fail(TQ_ERR_ARG, "tq_append_token: dtype must be TQ_F32 or TQ_BF16");
  if (ctx->d != 128) return fail(TQ_ERR_UNSUPPORTED, "tq_append_token: d must be 128");
  if (cache->host_max_len + 1 > cache->capacity) return fail(TQ_ERR_CAPACITY, "tq_append_token: cache is full");
  if ((s = check_device(ctx, fn)) != TQ_OK) return s;
  hipError_t e = launch_append(ctx, cache, d_k, d_v, dtype == TQ_BF16, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, fn);
  cache->host_max_len += 1;
  return TQ_OK;
}

size_t tq_attention_decode_ws_bytes(const tq_ctx *ctx, const tq_kv_cache *cache, int32_t q_heads) {
  if (!ctx || !cache || q_heads <= 0 || cache->kv_heads <= 0 || (q_heads % cache->kv_heads) != 0) return 0;
  return decode_ws_bytes(ctx, cache, q_heads, nullptr, nullptr);
}

tq_status tq_attention_decode(const tq_ctx *ctx, const tq_kv_cache *cache, const void *d_q, tq_dtype dtype,
                              int32_t q_heads, float scale, float *d_out, void *d_ws, size_t ws_bytes,
                              void *stream) {
  const char *fn = "tq_attention_decode";
  hipEvent_t ev[2];
  take_decode_events(ev);
  if (!ctx) return fail(TQ_ERR_ARG, "tq_attention_decode: NULL ctx");
  tq_status s = check_cache(ctx, cache, fn);
  if (s != TQ_OK) return s;
  if (!d_q || !d_out) return fail(TQ_ERR_ARG, "tq_attention_decode: NULL query or output");
  if (dtype != TQ_F32 && dtype != TQ_BF16) return fail(TQ_ERR_ARG, "tq_attention_decode: dtype must be TQ_F32 or TQ_BF16");
  if (q_heads <= 0 || (q_heads % cache->kv_heads) != 0)
    return fail(TQ_ERR_ARG, "tq_attention_decode: q_heads must be a positive multiple of kv_heads");
  if (q_heads / cache->kv_heads > 16) return fail(TQ_ERR_UNSUPPORTED, "tq_attention_decode: at most 16 query heads per KV head");
  if (ctx->d != 128) return fail(TQ_ERR_UNSUPPORTED, "tq_attention_decode: d must be 128");
  if (!std::isfinite(scale)) return fail(TQ_ERR_ARG, "tq_attention_decode: scale must be finite");
  size_t need = tq_attention_decode_ws_bytes(ctx, cache, q_heads);
  if (!d_ws || ws_bytes < need) return fail(TQ_ERR_CAPACITY, "tq_attention_decode: workspace smaller than tq_attention_decode_ws_bytes()");
  if ((s = check_device(ctx, fn)) != TQ_OK) return s;
  hipError_t e = launch_decode(ctx, cache, d_q, dtype == TQ_BF16, q_heads, scale, d_out, d_ws, (hipStream_t)stream,
                               nullptr, nullptr, ev[0], ev[1]);
  return e == hipSuccess ? TQ_OK : hip_fail(e, fn);
}

tq_status tq_attention_decode_noalloc(const tq_ctx *ctx, const tq_kv_cache *cache, const void *d_q, tq_dtype dtype,
                                      int32_t q_heads, float scale, float *d_out, void *stream) {
  const char *fn = "tq_attention_decode_noalloc";
  hipEvent_t ev[2];
  take_decode_events(ev);
  if (!ctx) return fail(TQ_ERR_ARG, "tq_attention_decode_noalloc: NULL ctx");
  tq_status s = check_cache(ctx, cache, fn);
  if (s != TQ_OK) return s;
  if (!d_q || !d_out) return fail(TQ_ERR_ARG, "tq_attention_decode_noalloc: NULL query or output");
  if (dtype != TQ_F32 && dtype != TQ_BF16)
    return fail(TQ_ERR_ARG, "tq_attention_decode_noalloc: dtype must be TQ_F32 or TQ_BF16");
  if (q_heads <= 0 || (q_heads % cache->kv_heads) != 0)
    return fail(TQ_ERR_ARG, "tq_attention_decode_noalloc: q_heads must be a positive multiple of kv_heads");
  if (q_heads / cache->kv_heads > 16)
    return fail(TQ_ERR_UNSUPPORTED, "tq_attention_decode_noalloc: at most 16 query heads per KV head");
  if (ctx->d != 128) return fail(TQ_ERR_UNSUPPORTED, "tq_attention_decode_noalloc: d must be 128");
  if (!std::isfinite(scale)) return fail(TQ_ERR_ARG, "tq_attention_decode_noalloc: scale must be finite");
  const size_t need = tq_attention_decode_ws_bytes(ctx, cache, q_heads);
  if (need > (size_t)TQ_SCRATCH_BYTES)
    return fail(TQ_ERR_CAPACITY, "tq_attention_decode_noalloc: this call needs " + std::to_string(need) +
                                     " bytes of scratch, more than the library's TQ_SCRATCH_BYTES = " +
                                     std::to_string((size_t)TQ_SCRATCH_BYTES) +
                                     " (use tq_attention_decode with a caller workspace)");
  if ((s = check_device(ctx, fn)) != TQ_OK) return s;
  void *ws = scratch_ptr(ctx->device);
  if (!ws) return fail(TQ_ERR_HIP, "tq_attention_decode_noalloc: no scratch address for the context's device");
  hipError_t e = launch_decode(ctx, cache, d_q, dtype == TQ_BF16, q_heads, scale, d_out, ws, (hipStream_t)stream,
                               nullptr, nullptr, ev[0], ev[1]);
  return e == hipSuccess ? TQ_OK : hip_fail(e, fn);
}

tq_status tq_decode_logits(const tq_ctx *ctx, const tq_kv_cache *cache, const void *d_q, tq_dtype dtype,
                           int32_t q_heads, float scale, float *d_logits, void *d_ws, size_t ws_bytes, void *stream) {
  const char *fn = "tq_decode_logits";
  hipEvent_t ev[2];
  take_decode_events(ev);
  if (!ctx) return fail(TQ_ERR_ARG, "tq_decode_logits: NULL ctx");
  tq_status s = check_cache(ctx, cache, fn);
  if (s != TQ_OK) return s;
  if (!d_q || !d_logits) return fail(TQ_ERR_ARG, "tq_decode_logits: NULL query or output");
  if (dtype != TQ_F32 && dtype != TQ_BF16) return fail(TQ_ERR_ARG, "tq_decode_logits: dtype must be TQ_F32 or TQ_BF16");
  if (q_heads <= 0 || (q_heads % cache->kv_heads) != 0)
    return fail(TQ_ERR_ARG, "tq_decode_logits: q_heads must be a positive multiple of kv_heads");
  if (q_heads / cache->kv_heads > 16) return fail(TQ_ERR_UNSUPPORTED, "tq_decode_logits: at most 16 query heads per KV head");
  if (ctx->d != 128) return fail(TQ_ERR_UNSUPPORTED, "tq_decode_logits: d must be 128");
  if (cache->d_block_table) return fail(TQ_ERR_UNSUPPORTED, "tq_decode_logits: contiguous caches only");
  if (!std::isfinite(scale)) return fail(TQ_ERR_ARG, "tq_decode_logits: scale must be finite");
  size_t need = tq_attention_decode_ws_bytes(ctx, cache, q_heads);
  if (!d_ws || ws_bytes < need) return fail(TQ_ERR_CAPACITY, "tq_decode_logits: workspace smaller than tq_attention_decode_ws_bytes()");
  if ((s = check_device(ctx, fn)) != TQ_OK) return s;
  hipError_t e = launch_decode(ctx, cache, d_q, dtype == TQ_BF16, q_heads, scale, nullptr, d_ws, (hipStream_t)stream,
                               nullptr, nullptr, ev[0], ev[1], 1, 0, nullptr, 0, d_logits);
  return e == hipSuccess ? TQ_OK : hip_fail(e, fn);
}

size_t tq_attention_prefill_ws_bytes(const tq_ctx *ctx, const tq_kv_cache *cache, int32_t n_q, int32_t q_heads) {
  if (!ctx || !cache || n_q <= 0 || q_heads <= 0 || cache->kv_heads <= 0 || (q_heads % cache->kv_heads) != 0) return 0;
  if (prefill_supported(ctx, cache, q_heads, n_q)) return prefill_ws_bytes(cache, q_heads, n_q);
  return decode_ws_bytes(ctx, cache, q_heads, nullptr, nullptr, n_q);
}

tq_status tq_attention_prefill(const tq_ctx *ctx, const tq_kv_cache *cache, const void *d_q, tq_dtype dtype,
                               int32_t n_q, int32_t q_heads, int32_t causal, float scale, float *d_out, void *d_ws,
                               size_t ws_bytes, void *stream) {
  const char *fn = "tq_attention_prefill";
  hipEvent_t ev[2];
  take_decode_events(ev);
  if (!ctx) return fail(TQ_ERR_ARG, "tq_attention_prefill: NULL ctx");
  tq_status s = check_cache(ctx, cache, fn);
  if (s != TQ_OK) return s;
  if (!d_q || !d_out) return fail(TQ_ERR_ARG, "tq_attention_prefill: NULL query or output");
  if (dtype != TQ_F32 && dtype != TQ_BF16) return fail(TQ_ERR_ARG, "tq_attention_prefill: dtype must be TQ_F32 or TQ_BF16");
  if (n_q <= 0) return fail(TQ_ERR_ARG, "tq_attention_prefill: n_q must be positive");
  if (causal != 0 && causal != 1) return fail(TQ_ERR_ARG, "tq_attention_prefill: causal must be 0 or 1");
  if (q_heads <= 0 || (q_heads % cache->kv_heads) != 0)
    return fail(TQ_ERR_ARG, "tq_attention_prefill: q_heads must be a positive multiple of kv_heads");
  if (q_heads / cache->kv_heads > 16) return fail(TQ_ERR_UNSUPPORTED, "tq_attention_prefill: at most 16 query heads per KV head");
  if ((int64_t)n_q * (q_heads / cache->kv_heads) > (1 << 20))
    return fail(TQ_ERR_UNSUPPORTED, "tq_attention_prefill: at most 2^20 query heads per KV head");
  if (ctx->d != 128) return fail(TQ_ERR_UNSUPPORTED, "tq_attention_prefill: d must be 128");
  if (!std::isfinite(scale)) return fail(TQ_ERR_ARG, "tq_attention_prefill: scale must be finite");
  // contiguous caches with at least 16 virtual heads per KV head and values of
  // at most 3 bits: the prefill kernel (16 virtual heads per work-group);
  // otherwise the decode kernels over groups of 4 virtual heads
  const bool pf = prefill_supported(ctx, cache, q_heads, n_q);
  {
    // one 256-thread work-group per (chunk, KV stream, group of 4 or 16 virtual
    // heads): the 1-D grid must stay below 2^32 work-items
    int chunk = 0, nchunks = 0;
    decode_ws_bytes(ctx, cache, q_heads, &chunk, &nchunks, n_q);
    const int64_t units = (int64_t)cache->batch * cache->kv_heads * (((int64_t)n_q * (q_heads / cache->kv_heads) + 3) / 4);
    if (units * nchunks >= ((int64_t)1 << 24))
      return fail(TQ_ERR_UNSUPPORTED, "tq_attention_prefill: batch x query positions x context too large for one launch");
  }
  size_t need = tq_attention_prefill_ws_bytes(ctx, cache, n_q, q_heads);
  if (!d_ws || ws_bytes < need) return fail(TQ_ERR_CAPACITY, "tq_attention_prefill: workspace smaller than tq_attention_prefill_ws_bytes()");
  if ((s = check_device(ctx, fn)) != TQ_OK) return s;
  hipError_t e = pf ? launch_prefill(ctx, cache, d_q, dtype == TQ_BF16, q_heads, n_q, causal, scale, d_out, d_ws,
                                     (hipStream_t)stream, ev[0], ev[1])
                    : launch_decode(ctx, cache, d_q, dtype == TQ_BF16, q_heads, scale, d_out, d_ws, (hipStream_t)stream,
                                    nullptr, nullptr, ev[0], ev[1], n_q, causal);
  return e == hipSuccess ? TQ_OK : hip_fail(e, fn);
}

size_t tq_decode_step_ws_bytes(const tq_ctx *ctx, const tq_kv_cache *cache, int32_t q_heads) {
  if (!ctx || !cache || q_heads <= 0 || cache->kv_heads <= 0 || (q_heads % cache->kv_heads) != 0) return 0;
  tq_kv_cache after = *cache;
  after.host_max_len = std::min(cache->host_max_len + 1, cache->capacity);
  return decode_ws_bytes(ctx, &after, q_heads, nullptr, nullptr);
}

tq_status tq_decode_step(const tq_ctx *ctx, tq_kv_cache *cache, const void *d_k, const void *d_v, const void *d_q,
                         tq_dtype dtype, int32_t q_heads, float scale, float *d_out, void *d_ws, size_t ws_bytes,
                         void *stream) {
  const char *fn = "tq_decode_step";
  hipEvent_t ev[2];
  take_decode_events(ev);
  if (!ctx) return fail(TQ_ERR_ARG, "tq_decode_step: NULL ctx");
  tq_status s = check_cache(ctx, cache, fn);
  if (s != TQ_OK) return s;
  if (!d_k || !d_v || !d_q || !d_out) return fail(TQ_ERR_ARG, "tq_decode_step: NULL input or output");
  if (dtype != TQ_F32 && dtype != TQ_BF16) return fail(TQ_ERR_ARG, "tq_decode_step: dtype must be TQ_F32 or TQ_BF16");
  if (q_heads <= 0 || (q_heads % cache->kv_heads) != 0)
    return fail(TQ_ERR_ARG, "tq_decode_step: q_heads must be a positive multiple of kv_heads");
  if (q_heads / cache->kv_heads > 16) return fail(TQ_ERR_UNSUPPORTED, "tq_decode_step: at most 16 query heads per KV head");
  if (ctx->d != 128) return fail(TQ_ERR_UNSUPPORTED, "tq_decode_step: d must be 128");
  if (!std::isfinite(scale)) return fail(TQ_ERR_ARG, "tq_decode_step: scale must be finite");
  if (cache->host_max_len + 1 > cache->capacity) return fail(TQ_ERR_CAPACITY, "tq_decode_step: cache is full");
  size_t need = tq_decode_step_ws_bytes(ctx, cache, q_heads);
  if (!d_ws || ws_bytes < need) return fail(TQ_ERR_CAPACITY, "tq_decode_step: workspace smaller than tq_decode_step_ws_bytes()");
  if ((s = check_device(ctx, fn)) != TQ_OK) return s;
  tq_kv_cache after = *cache;
  after.host_max_len = cache->host_max_len + 1;
  hipError_t e = launch_decode(ctx, &after, d_q, dtype == TQ_BF16, q_heads, scale, d_out, d_ws, (hipStream_t)stream,
                               d_k, d_v, ev[0], ev[1]);
  if (e != hipSuccess) return hip_fail(e, fn);
  cache->host_max_len += 1;
  return TQ_OK;
}

static tq_status check_polar(const tq_ctx *ctx, const tq_polar_packed *p, const char *fn) {
  if (ctx->d != 128) return fail(TQ_ERR_UNSUPPORTED, std::string(fn) + ": the PolarQuant path needs d = 128");
  if (!p || !p->bits || !p->norms) return fail(TQ_ERR_ARG, std::string(fn) + ": packed array or its pointers NULL");
  if (p->b1 < 1 || p->b1 > TQ_MAX_BITS || p->b2 < 1 || p->b2 > TQ_MAX_BITS)
    return fail(TQ_ERR_UNSUPPORTED, std::string(fn) + ": b1 and b2 must be in [1, 4]");
  if (p->n < 0) return fail(TQ_ERR_ARG, std::string(fn) + ": negative record count");
  return TQ_OK;
}

size_t tq_polar_quantize_ws_bytes(const tq_ctx *ctx, int64_t n) {
  if (!ctx || n < 0) return 0;
  return (size_t)n * ctx->d * sizeof(float) + 256;
}

tq_status tq_polar_quantize(const tq_ctx *ctx, const void *d_x, tq_dtype dtype, int64_t n_streams, int64_t n_tokens,
                            int64_t x_stride, const tq_polar_packed *out, int64_t out_stream_stride,
                            int64_t out_offset, void *d_ws, size_t ws_bytes, void *stream) {
  const char *fn = "tq_polar_quantize";
  if (!ctx) return fail(TQ_ERR_ARG, "tq_polar_quantize: NULL ctx");
  tq_status s = check_polar(ctx, out, fn);
  if (s != TQ_OK) return s;
  if (dtype != TQ_F32 && dtype != TQ_BF16) return fail(TQ_ERR_ARG, "tq_polar_quantize: dtype must be TQ_F32 or TQ_BF16");
  if (n_streams < 0 || n_tokens < 0 || out_offset < 0 || x_stride < 0 || out_stream_stride < 0)
    return fail(TQ_ERR_ARG, "tq_polar_quantize: negative size, stride or offset");
  if (n_streams == 0 || n_tokens == 0) return TQ_OK;
  if (!d_x) return fail(TQ_ERR_ARG, "tq_polar_quantize: NULL input");
  if (x_stride < ctx->d || (x_stride % 8) != 0 || ((uintptr_t)d_x % 16) != 0)
    return fail(TQ_ERR_ARG, "tq_polar_quantize: input must be 16-byte aligned with a row stride >= d, a multiple of 8");
  if (n_streams > 1 && out_stream_stride < out_offset + n_tokens)
    return fail(TQ_ERR_ARG, "tq_polar_quantize: output streams overlap (out_stream_stride < out_offset + n_tokens)");
  if ((n_streams - 1) * out_stream_stride + out_offset + n_tokens > out->n)
    return fail(TQ_ERR_ARG, "tq_polar_quantize: records past the end of the output array");
  const int64_t n = n_streams * n_tokens;
  if ((n + 3) / 4 > INT32_MAX || (n + 63) / 64 > INT32_MAX)
    return fail(TQ_ERR_UNSUPPORTED, "tq_polar_quantize: too many vectors for one launch");
  if (!d_ws || ws_bytes < tq_polar_quantize_ws_bytes(ctx, n))
    return fail(TQ_ERR_CAPACITY, "tq_polar_quantize: workspace smaller than tq_polar_quantize_ws_bytes()");
  if ((s = check_device(ctx, fn)) != TQ_OK) return s;
  hipError_t e = launch_polar_quantize(ctx, d_x, dtype == TQ_BF16, n_streams, n_tokens, x_stride, out,
                                       out_stream_stride, out_offset, d_ws, (hipStream_t)stream);
  return e == hipSuccess ? TQ_OK : hip_fail(e, fn);
}

size_t tq_polar_attention_decode_ws_bytes(const tq_ctx *ctx, const tq_kv_cache *values, int32_t q_heads) {
  if (!ctx || !values || q_heads <= 0 || values->kv_heads <= 0 || (q_heads % values->kv_heads) != 0) return 0;
  return polar_attention_ws_bytes(ctx, values, q_heads);
}

tq_status tq_polar_attention_decode(const tq_ctx *ctx, const tq_polar_packed *keys, const tq_kv_cache *values,
                                    const void *d_q, tq_dtype dtype, int32_t q_heads, float scale, float *d_out,
                                    void *d_ws, size_t ws_bytes, void *stream) {
  const char *fn = "tq_polar_attention_decode";
  hipEvent_t ev[2];
  take_decode_events(ev);
  if (!ctx) return fail(TQ_ERR_ARG, "tq_polar_attention_decode: NULL ctx");
  tq_status s = check_polar(ctx, keys, fn);
  if (s != TQ_OK) return s;
  if (!values) return fail(TQ_ERR_ARG, "tq_polar_attention_decode: NULL values");
  if ((s = check_packed(ctx, &values->v, 0, fn)) != TQ_OK) return s;
  if (values->batch <= 0 || values->kv_heads <= 0 || values->capacity <= 0 || (values->capacity % 32) != 0)
    return fail(TQ_ERR_ARG, "tq_polar_attention_decode: batch, kv_heads > 0 and capacity a positive multiple of 32 required");
  if (values->d_block_table || values->v.norm_f16)
    return fail(TQ_ERR_UNSUPPORTED, "tq_polar_attention_decode: contiguous values with fp32 norms only");
  const int64_t recs = (int64_t)values->batch * values->kv_heads * values->capacity;
  if (values->v.n < recs || keys->n < recs)
    return fail(TQ_ERR_ARG, "tq_polar_attention_decode: key or value records fewer than batch*kv_heads*capacity");
  if (!values->d_seq_len) return fail(TQ_ERR_ARG, "tq_polar_attention_decode: NULL d_seq_len");
  if (values->host_max_len < 0 || values->host_max_len > values->capacity)
    return fail(TQ_ERR_ARG, "tq_polar_attention_decode: host_max_len outside [0, capacity]");
  if (!d_q || !d_out) return fail(TQ_ERR_ARG, "tq_polar_attention_decode: NULL query or output");
  if (dtype != TQ_F32 && dtype != TQ_BF16) return fail(TQ_ERR_ARG, "tq_polar_attention_decode: dtype must be TQ_F32 or TQ_BF16");
  if (((uintptr_t)d_q % 16) != 0) return fail(TQ_ERR_ARG, "tq_polar_attention_decode: queries must be 16-byte aligned");
  if (q_heads <= 0 || (q_heads % values->kv_heads) != 0)
    return fail(TQ_ERR_ARG, "tq_polar_attention_decode: q_heads must be a positive multiple of kv_heads");
  if (q_heads / values->kv_heads > 16) return fail(TQ_ERR_UNSUPPORTED, "tq_polar_attention_decode: at most 16 query heads per KV head");
  if ((int64_t)values->batch * values->kv_heads * ((q_heads / values->kv_heads + 3) / 4) > 65535)
    return fail(TQ_ERR_UNSUPPORTED, "tq_polar_attention_decode: at most 65535 (stream, head group) units");
  if (!std::isfinite(scale)) return fail(TQ_ERR_ARG, "tq_polar_attention_decode: scale must be finite");
  if (!d_ws || ws_bytes < tq_polar_attention_decode_ws_bytes(ctx, values, q_heads))
    return fail(TQ_ERR_CAPACITY, "tq_polar_attention_decode: workspace smaller than tq_polar_attention_decode_ws_bytes()");
  if ((s = check_device(ctx, fn)) != TQ_OK) return s;
  hipError_t e = launch_polar_attention(ctx, keys, values, d_q, dtype == TQ_BF16, q_heads, scale, d_out, d_ws,
                                        (hipStream_t)stream, ev[0], ev[1]);
  return e == hipSuccess ? TQ_OK : hip_fail(e, fn);
}

size_t tq_polar_scores_ws_bytes(const tq_ctx *ctx, int64_t nq, int64_t n) {
  if (!ctx || nq < 0 || n < 0) return 0;
  return (((size_t)nq * ctx->d * sizeof(float) + 255) & ~(size_t)255) + (size_t)n * ctx->d * sizeof(float) + 256;
}

tq_status tq_polar_scores(const tq_ctx *ctx, const void *d_q, tq_dtype dtype, int64_t nq, const tq_polar_packed *keys,
                          float *d_scores, void *d_ws, size_t ws_bytes, void *stream) {
  const char *fn = "tq_polar_scores";
  if (!ctx) return fail(TQ_ERR_ARG, "tq_polar_scores: NULL ctx");
  tq_status s = check_polar(ctx, keys, fn);
  if (s != TQ_OK) return s;
  if (dtype != TQ_F32 && dtype != TQ_BF16) return fail(TQ_ERR_ARG, "tq_polar_scores: dtype must be TQ_F32 or TQ_BF16");
  if (nq < 0) return fail(TQ_ERR_ARG, "tq_polar_scores: negative query count");
  if (nq == 0 || keys->n == 0) return TQ_OK;
  if (!d_q || !d_scores) return fail(TQ_ERR_ARG, "tq_polar_scores: NULL query or output");
  if (((uintptr_t)d_q % 16) != 0) return fail(TQ_ERR_ARG, "tq_polar_scores: queries must be 16-byte aligned");
  if ((keys->n + 3) / 4 > INT32_MAX || (keys->n + 127) / 128 > 65535 || (nq + 63) / 64 > INT32_MAX)
    return fail(TQ_ERR_UNSUPPORTED, "tq_polar_scores: too many keys for one launch (at most 8388480)");
  if (!d_ws || ws_bytes < tq_polar_scores_ws_bytes(ctx, nq, keys->n))
    return fail(TQ_ERR_CAPACITY, "tq_polar_scores: workspace smaller than tq_polar_scores_ws_bytes()");
  if ((s = check_device(ctx, fn)) != TQ_OK) return s;
  hipError_t e = launch_polar_scores(ctx, d_q, dtype == TQ_BF16, nq, keys, d_scores, d_ws, (hipStream_t)stream);
  return e == hipSuccess ? TQ_OK : hip_fail(e, fn);
}

size_t tq_scores_ws_bytes(const tq_ctx *ctx, int64_t nq, int64_t n, int32_t topk, int32_t want_scores) {
  if (!ctx || nq <= 0 || n <= 0 || topk < 0) return 0;
  return scores_ws_bytes(ctx, nq, n, topk, want_scores);
}

tq_status tq_scores(const tq_ctx *ctx, const void *d_q, tq_dtype dtype, int64_t nq, const tq_packed *keys,
                    float *d_scores, int32_t topk, int32_t *d_top_idx, float *d_top_val, void *d_ws,
                    size_t ws_bytes, void *stream) {
  const char *fn = "tq_scores";
  if (!ctx) return fail(TQ_ERR_ARG, "tq_scores: NULL ctx");
  tq_status s = check_packed(ctx, keys, 1, fn);
  if (s != TQ_OK) return s;
  if (dtype != TQ_F32 && dtype != TQ_BF16) return fail(TQ_ERR_ARG, "tq_scores: dtype must be TQ_F32 or TQ_BF16");
  if (nq < 0 || topk < 0) return fail(TQ_ERR_ARG, "tq_scores: negative nq or topk");
  if (topk > 64) return fail(TQ_ERR_UNSUPPORTED, "tq_scores: topk must be <= 64");
  if (topk > keys->n) return fail(TQ_ERR_ARG, "tq_scores: topk larger than the number of keys");
  if (!d_scores && topk == 0) return fail(TQ_ERR_ARG, "tq_scores: nothing requested (no scores, topk = 0)");
  if (topk > 0 && (!d_top_idx || !d_top_val)) return fail(TQ_ERR_ARG, "tq_scores: NULL top-k output");
  if (nq == 0 || keys->n == 0) return TQ_OK;
  if (!d_q) return fail(TQ_ERR_ARG, "tq_scores: NULL queries");
  if (((uintptr_t)d_q % 16) != 0) return fail(TQ_ERR_ARG, "tq_scores: queries must be 16-byte aligned");
  if ((keys->n + 127) / 128 > 65535 * 1024LL) return fail(TQ_ERR_UNSUPPORTED, "tq_scores: too many keys");
  size_t need = scores_ws_bytes(ctx, nq, keys->n, topk, d_scores != nullptr);
  if (!d_ws || ws_bytes < need) return fail(TQ_ERR_CAPACITY, "tq_scores: workspace smaller than tq_scores_ws_bytes()");
  if ((s = check_device(ctx, fn)) != TQ_OK) return s;
  hipError_t e = launch_scores(ctx, d_q, dtype == TQ_BF16, nq, keys, d_scores, topk, d_top_idx, d_top_val, d_ws,
                               (hipStream_t)stream);
  return e == hipSuccess ? TQ_OK : hip_fail(e, fn);
}

}  // extern "C"
