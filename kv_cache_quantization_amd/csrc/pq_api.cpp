// C ABI of the codec library: argument validation, the Lloyd-Max codebook,
// the search-grid geometry and kernel launches.  See include/pq.h for the
// contract of every entry point.
#include "../../include/pq.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <map>
#include <mutex>
#include <vector>

#include "pq_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return PQ_OK;
  g_last_hip_error = (int)e;
  return PQ_EHIP;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

int check_d(int d) {
  if (!is_pow2(d)) return PQ_EINVAL;
  if (d < 64 || d > 512) return PQ_EUNSUPPORTED;
  return PQ_OK;
}

// ------------------------------------------------------------------------------------------
// Lloyd-Max quantizer for N(0,1) (eliza quantization README, PolarQuant, "Algorithm in one
// paragraph"): centroids are the conditional means of their cells, boundaries the
// midpoints of adjacent centroids; iterated in double to a fixed point.  The start is the
// high-resolution optimum (point density proportional to pdf^(1/3), i.e. centroids at the
// quantiles of N(0, 3)), which is close to the fixed point for every bit width.
// ------------------------------------------------------------------------------------------
struct Codebook {
  std::vector<double> c, beta;
  double mse = 0.0;
};

double gauss_pdf(double x) { return std::exp(-0.5 * x * x) * 0.3989422804014327; }

// P(lo < X <= hi) for X ~ N(0,1), accurate in both tails
double gauss_mass(double lo, double hi) {
  const double k = 0.7071067811865476;
  if (lo >= 0.0) return 0.5 * (std::erfc(lo * k) - std::erfc(hi * k));
  if (hi <= 0.0) return 0.5 * (std::erfc(-hi * k) - std::erfc(-lo * k));
  return 1.0 - 0.5 * std::erfc(-lo * k) - 0.5 * std::erfc(hi * k);
}

double gauss_quantile(double p) {
  double lo = -40.0, hi = 40.0;
  for (int it = 0; it < 200; ++it) {
    const double mid = 0.5 * (lo + hi);
    if (gauss_mass(-INFINITY, mid) < p) lo = mid; else hi = mid;
  }
  return 0.5 * (lo + hi);
}

Codebook solve_codebook(int bits) {
  const int L = 1 << bits;
  Codebook cb;
  cb.c.resize(L);
  for (int k = 0; k < L; ++k) cb.c[k] = std::sqrt(3.0) * gauss_quantile((k + 0.5) / L);
  std::vector<double> beta(L - 1), cn(L), mass(L);
  for (int it = 0; it < 4000000; ++it) {
    for (int k = 0; k + 1 < L; ++k) beta[k] = 0.5 * (cb.c[k] + cb.c[k + 1]);
    double step = 0.0;
    for (int k = 0; k < L; ++k) {
      const double lo = k == 0 ? -INFINITY : beta[k - 1];
      const double hi = k == L - 1 ? INFINITY : beta[k];
      mass[k] = gauss_mass(lo, hi);
      const double num = (k == 0 ? 0.0 : gauss_pdf(lo)) - (k == L - 1 ? 0.0 : gauss_pdf(hi));
      cn[k] = num / mass[k];
      step = std::max(step, std::fabs(cn[k] - cb.c[k]));
    }
    cb.c.swap(cn);
    if (step < 1e-13) break;
  }
  for (int k = 0; k < L / 2; ++k) {            // exact symmetry of the N(0,1) fixed point
    const double v = 0.5 * (cb.c[L - 1 - k] - cb.c[k]);
    cb.c[k] = -v;
    cb.c[L - 1 - k] = v;
  }
  cb.beta.resize(L - 1);
  for (int k = 0; k + 1 < L; ++k) cb.beta[k] = 0.5 * (cb.c[k] + cb.c[k + 1]);
  double acc = 0.0;
  for (int k = 0; k < L; ++k) {
    const double lo = k == 0 ? -INFINITY : cb.beta[k - 1];
    const double hi = k == L - 1 ? INFINITY : cb.beta[k];
    acc += gauss_mass(lo, hi) * cb.c[k] * cb.c[k];
  }
  cb.mse = 1.0 - acc;
  return cb;
}

std::once_flag g_cb_once[pqi::kMaxBits + 1];
Codebook g_cb[pqi::kMaxBits + 1];

const Codebook& codebook(int bits) {
  std::call_once(g_cb_once[bits], [bits] { g_cb[bits] = solve_codebook(bits); });
  return g_cb[bits];
}

// fp32 tables and search-grid geometry for the kernels
pqi::CodecTables build_tables(int bits);

std::once_flag g_tab_once[pqi::kMaxBits + 1];
pqi::CodecTables g_tab[pqi::kMaxBits + 1];

// built once per bit width (the codebook and grid never change)
const pqi::CodecTables& make_tables(int bits) {
  std::call_once(g_tab_once[bits], [bits] { g_tab[bits] = build_tables(bits); });
  return g_tab[bits];
}

pqi::CodecTables build_tables(int bits) {
  const Codebook& cb = codebook(bits);
  pqi::CodecTables t;
  std::memset(&t, 0, sizeof(t));
  const int L = 1 << bits;
  for (int k = 0; k < L; ++k) t.cent[k] = (float)cb.c[k];
  for (int k = 0; k + 1 < L; ++k) t.beta[k] = (float)cb.beta[k];
  t.nbound = L - 1;
  double w, Y;
  if (L == 2) {
    w = 0.5;
    Y = 2.0;
  } else {
    // a cell narrower than the smallest boundary gap holds at most one boundary, and the
    // boundary nearest to its centre decides every y that rounds into it
    double gap = INFINITY;
    for (int k = 0; k + 2 < L; ++k) gap = std::min(gap, (double)t.beta[k + 1] - (double)t.beta[k]);
    w = 0.9 * gap;
    Y = (double)t.beta[L - 2] + w;
  }
  t.half = (int)std::ceil(Y / w);
  t.ncell = 2 * t.half + 1;
  // nearest boundary to each cell centre (k - half) w, as the kernels compute it in fp32
  for (int k = 0; k < t.ncell; ++k) {
    const float c = (float)(k - t.half) * (float)w;
    int best = 0;
    float bd = std::fabs(t.beta[0] - c);
    for (int j = 1; j < t.nbound; ++j) {
      const float dd = std::fabs(t.beta[j] - c);
      if (dd < bd) { bd = dd; best = j; }
    }
    t.cell_best[k] = (uint8_t)best;
  }
  // one copy of the grid per lane of a 16-lane LDS access group when it fits in 64 KiB
  t.nrep = (size_t)t.ncell * 16 * 16 <= 65536 ? 16 : 1;
  t.cell_w = (float)w;
  t.cell_inv_w = (float)(1.0 / w);
  return t;
}

// CU count and LDS limit of the current device, read once per device
constexpr int kCfgDevices = 64;
std::mutex g_cfg_mu;
pqi::LaunchCfg g_cfg[kCfgDevices];
bool g_cfg_ok[kCfgDevices] = {};

int launch_cfg(pqi::LaunchCfg* c) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  const bool cached = dev >= 0 && dev < kCfgDevices;
  if (cached) {
    std::lock_guard<std::mutex> lock(g_cfg_mu);
    if (g_cfg_ok[dev]) {
      *c = g_cfg[dev];
      return PQ_OK;
    }
  }
  e = hipDeviceGetAttribute(&c->cu_count, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_status(e);
  e = hipDeviceGetAttribute(&c->max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  if (e != hipSuccess) return hip_status(e);
  if (cached) {
    std::lock_guard<std::mutex> lock(g_cfg_mu);
    g_cfg[dev] = *c;
    g_cfg_ok[dev] = true;
  }
  return PQ_OK;
}

constexpr int64_t kMaxElems = INT64_MAX / 8;

// ------------------------------------------------------------------------------------------
// Seeded rotation signs and JL matrix (eliza quantization README, TurboQuant "CLI": layer i
// uses seed base_seed + i; QJL "CLI": --projection-seed).  A counter-based generator, so that
// any consumer rebuilds the same bytes from the seed: SplitMix64 (Steele, Lea and Flood,
// OOPSLA 2014), stream (seed, tag) started in state mix(seed ^ tag), output i =
// mix(state + (i + 1) * golden gamma); signs from the top bit of each output; Gaussians by the
// Box-Muller transform of output pairs taken as uniforms in (0, 1), rounded to bf16.
// ------------------------------------------------------------------------------------------
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kTagSigns = 0x5349474Eull;   // "SIGN"
constexpr uint64_t kTagProj = 0x50524F4Aull;    // "PROJ"

uint64_t splitmix_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

struct SeedStream {
  uint64_t state;
  SeedStream(uint64_t seed, uint64_t tag) : state(splitmix_mix(seed ^ tag)) {}
  uint64_t next() { return splitmix_mix(state += kGamma); }
};

// uniform in (0, 1) from the top 53 bits: ((z >> 11) + 1/2) 2^-53
double unit_open(uint64_t z) { return ((double)(z >> 11) + 0.5) * 0x1p-53; }

// double -> bf16 bits, round to nearest even, directly from the double (no fp32 step, which
// would round twice); overflow to infinity, NaN to a quiet NaN.
uint16_t bf16_rne(double v) {
  uint64_t b;
  std::memcpy(&b, &v, sizeof(b));
  const uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  const double a = std::fabs(v);
  if (std::isnan(v)) return (uint16_t)(sign | 0x7FC0u);
  if (a < 0x1p-126) {                      // bf16 subnormal range: quantum 2^-133
    const double q = std::nearbyint(a * 0x1p133);
    return (uint16_t)(sign | (uint16_t)q);  // q <= 128; 128 is the smallest normal
  }
  uint64_t m = b & 0x7FFFFFFFFFFFFFFFull;
  m += (1ull << 44) - 1 + ((m >> 45) & 1);   // 45 dropped fraction bits, ties to even
  m >>= 45;                                  // (double exponent << 7) | 7 fraction bits
  const int64_t e = (int64_t)(m >> 7) - 1023 + 127;
  if (e >= 255) return (uint16_t)(sign | 0x7F80u);
  return (uint16_t)(sign | (uint16_t)((e << 7) | (int64_t)(m & 0x7F)));
}

}  // namespace

namespace {

int quantize_impl(int d, int bits, int in_dtype, const void* x, int64_t n_blocks, const uint8_t* signs, int m,
                  const uint16_t* proj, uint8_t* codes, uint16_t* norms, uint8_t* qjl_bits, uint16_t* rnorms,
                  int pbits, void* stream) {
  int st = check_d(d);
  if (st) return st;
  if (bits < 1 || bits > pqi::kMaxBits) return PQ_EINVAL;
  if (in_dtype != PQ_F32 && in_dtype != PQ_BF16) return PQ_EINVAL;
  if (n_blocks < 0 || n_blocks > kMaxElems / d) return PQ_EINVAL;
  if (m < 0 || (m % 8) != 0) return PQ_EINVAL;
  if (m > 1024) return PQ_EUNSUPPORTED;
  if (m == 0 && (proj || qjl_bits || rnorms)) return PQ_EINVAL;
  if (n_blocks == 0) return PQ_OK;
  if (!x || !signs || !codes || !norms) return PQ_EINVAL;
  if (m > 0 && (!proj || !qjl_bits || !rnorms)) return PQ_EINVAL;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(norms, 2)) return PQ_EINVAL;
  if (m > 0 && (!aligned(proj, 16) || !aligned(qjl_bits, 16) || !aligned(rnorms, 2))) return PQ_EINVAL;
  pqi::LaunchCfg cfg;
  if ((st = launch_cfg(&cfg))) return st;
  pqi::QuantArgs a;
  a.x = x; a.n_blocks = n_blocks; a.signs = signs; a.proj = proj; a.codes = codes; a.norms = norms;
  a.qbits = qjl_bits; a.rnorms = rnorms; a.m = m; a.pbits = pbits; a.t = make_tables(bits);
  return hip_status(pqi::launch_quantize(d, in_dtype == PQ_BF16, a, cfg, (hipStream_t)stream));
}

int dequantize_impl(int d, int bits, const uint8_t* codes, const uint16_t* norms, int64_t n_blocks,
                    const uint8_t* signs, int out_dtype, void* out, int pbits, void* stream) {
  int st = check_d(d);
  if (st) return st;
  if (bits < 1 || bits > pqi::kMaxBits) return PQ_EINVAL;
  if (out_dtype != PQ_F32 && out_dtype != PQ_BF16) return PQ_EINVAL;
  if (n_blocks < 0 || n_blocks > kMaxElems / d) return PQ_EINVAL;
  if (n_blocks == 0) return PQ_OK;
  if (!codes || !norms || !signs || !out) return PQ_EINVAL;
  if (!aligned(codes, 16) || !aligned(out, 16) || !aligned(norms, 2)) return PQ_EINVAL;
  pqi::LaunchCfg cfg;
  if ((st = launch_cfg(&cfg))) return st;
  pqi::DequantArgs a;
  a.codes = codes; a.norms = norms; a.n_blocks = n_blocks; a.signs = signs; a.out = out; a.pbits = pbits;
  a.t = make_tables(bits);
  return hip_status(pqi::launch_dequantize(d, out_dtype == PQ_BF16, a, cfg, (hipStream_t)stream));
}

// Lloyd-Max quantizer of one coordinate of a uniform unit vector in R^d (eliza quantization
// README, TurboQuant, "Algorithm in one paragraph": the coordinates after a random rotation
// follow this law, and the codes use its Lloyd-Max centroids).  Density
// f(t) = K (1 - t^2)^((d-3)/2) on (-1, 1); the distribution function comes from a fine
// trapezoid table (2^21 steps), the first moment of a cell in closed form,
// int t f = -K (1 - t^2)^((d-1)/2) / (d - 1); iterated to a fixed point and made exactly
// antisymmetric (the law is symmetric).
struct SphereTable {
  std::vector<double> cdf;   // at t_i = -1 + 2 i / n
  double K = 0.0;
  int d = 0;
};

Codebook solve_sphere_codebook(int bits, int d) {
  const int n = 1 << 21;
  SphereTable tb;
  tb.d = d;
  tb.K = std::exp(std::lgamma(d / 2.0) - std::lgamma((d - 1) / 2.0)) / std::sqrt(M_PI);
  tb.cdf.resize(n + 1);
  const double h = 2.0 / n, ex = (d - 3) / 2.0;
  auto f = [&](double t) { const double u = 1.0 - t * t; return u > 0.0 ? tb.K * std::pow(u, ex) : 0.0; };
  double acc = 0.0, prev = f(-1.0);
  tb.cdf[0] = 0.0;
  for (int i = 1; i <= n; ++i) {
    const double cur = f(-1.0 + h * i);
    acc += 0.5 * h * (prev + cur);
    tb.cdf[i] = acc;
    prev = cur;
  }
  for (int i = 0; i <= n; ++i) tb.cdf[i] /= acc;          // the table's own normalisation
  auto cdf = [&](double t) {
    if (t <= -1.0) return 0.0;
    if (t >= 1.0) return 1.0;
    const double x = (t + 1.0) / h;
    const int i = std::min(n - 1, (int)x);
    const double w = x - i;
    return tb.cdf[i] * (1.0 - w) + tb.cdf[i + 1] * w;
  };
  auto mom = [&](double t) {
    const double u = std::max(0.0, 1.0 - t * t);
    return -tb.K * std::pow(u, (d - 1) / 2.0) / (d - 1);
  };
  const int L = 1 << bits;
  std::vector<double> beta(L - 1), c(L);
  for (int k = 0; k + 1 < L; ++k) {                      // equal-mass start
    double lo = -1.0, hi = 1.0;
    const double q = (double)(k + 1) / L;
    for (int it = 0; it < 200; ++it) {
      const double mid = 0.5 * (lo + hi);
      (cdf(mid) < q ? lo : hi) = mid;
    }
    beta[k] = 0.5 * (lo + hi);
  }
  auto cells = [&]() {
    for (int k = 0; k < L; ++k) {
      const double a = k ? beta[k - 1] : -1.0, b = k + 1 < L ? beta[k] : 1.0;
      c[k] = (mom(b) - mom(a)) / (cdf(b) - cdf(a));
    }
  };
  for (int it = 0; it < 200000; ++it) {
    cells();
    double change = 0.0;
    for (int k = 0; k + 1 < L; ++k) {
      const double nb = 0.5 * (c[k] + c[k + 1]);
      change = std::max(change, std::fabs(nb - beta[k]));
      beta[k] = nb;
    }
    if (change < 1e-13) break;
  }
  for (int k = 0; k < (L - 1) / 2; ++k) {
    const double v = 0.5 * (beta[L - 2 - k] - beta[k]);
    beta[k] = -v;
    beta[L - 2 - k] = v;
  }
  if (L > 2) beta[(L - 2) / 2] = 0.0;
  if (L == 2) beta[0] = 0.0;
  cells();
  for (int k = 0; k < L / 2; ++k) {
    const double v = 0.5 * (c[L - 1 - k] - c[k]);
    c[k] = -v;
    c[L - 1 - k] = v;
  }
  Codebook cb;
  cb.c = c;
  cb.beta = beta;
  return cb;
}

const Codebook& sphere_codebook(int bits, int d) {
  static std::mutex mu;
  static std::map<std::pair<int, int>, Codebook> cache;
  std::lock_guard<std::mutex> lock(mu);
  auto key = std::make_pair(bits, d);
  auto it = cache.find(key);
  if (it == cache.end()) it = cache.emplace(key, solve_sphere_codebook(bits, d)).first;
  return it->second;
}

int check_d_dense(int d) {
  if (d <= 0 || (d % 16) != 0) return PQ_EINVAL;
  if (d > pqi::kDenseMaxD) return PQ_EUNSUPPORTED;
  return PQ_OK;
}

// block-diagonal rotation: d a multiple of 32 in [64, 4096]
int check_d_bd(int d) {
  if (d <= 0 || (d % 32) != 0) return PQ_EINVAL;
  if (d < pqi::kBdMinD || d > pqi::kBdMaxD) return PQ_EUNSUPPORTED;
  return PQ_OK;
}

void fill_bd_codebook(int bits, pqi::BdArgs& a) {
  const Codebook& cb = codebook(bits);
  for (int k = 0; k < (1 << bits); ++k) a.cent[k] = (float)cb.c[k];
  for (int k = 0; k + 1 < (1 << bits); ++k) a.beta[k] = (float)cb.beta[k];
  const pqi::CodecTables& t = make_tables(bits);
  // a grid of at most 32 two-word cells sits in distinct LDS banks without copies per lane
  a.ncell = t.ncell; a.half = t.half; a.nrep = t.ncell <= 32 ? 1 : t.nrep;
  a.cell_w = t.cell_w; a.cell_inv_w = t.cell_inv_w;
}

}  // namespace

extern "C" {

int pq_abi_version(void) { return PQ_ABI_VERSION; }

const char* pq_strerror(int status) {
  switch (status) {
    case PQ_OK: return "ok";
    case PQ_EINVAL: return "invalid argument (pointer, size, alignment, dtype or parameter)";
    case PQ_EUNSUPPORTED: return "unsupported parameter combination";
    case PQ_EHIP: return "HIP runtime error (see pq_last_hip_error)";
    case PQ_ETOOBIG: return "request needs more work memory than the library's fixed work array";
  }
  return "unknown status";
}

int pq_last_hip_error(void) { return g_last_hip_error; }

int pq_make_signs(uint64_t seed, int d, uint8_t* mask) {
  if (d < 8 || d > 65536 || (d % 8) != 0 || !mask) return PQ_EINVAL;
  SeedStream s(seed, kTagSigns);
  std::memset(mask, 0, (size_t)d / 8);
  for (int j = 0; j < d; ++j)
    if (s.next() >> 63) mask[j >> 3] |= (uint8_t)(1u << (j & 7));
  return PQ_OK;
}

int qjl_make_projection(uint64_t seed, int m, int d, uint16_t* proj) {
  if (m < 1 || d < 1 || m > 65536 || d > 65536 || ((int64_t)m * d) % 2 != 0 || !proj) return PQ_EINVAL;
  SeedStream s(seed, kTagProj);
  const int64_t n = (int64_t)m * d;
  for (int64_t k = 0; k < n; k += 2) {
    const double u1 = unit_open(s.next());
    const double u2 = unit_open(s.next());
    const double rad = std::sqrt(-2.0 * std::log(u1));
    const double th = 2.0 * M_PI * u2;
    proj[k] = bf16_rne(rad * std::cos(th));
    proj[k + 1] = bf16_rne(rad * std::sin(th));
  }
  return PQ_OK;
}

int pq_codebook(int bits, double* centroids, double* boundaries, double* mse) {
  if (bits < 1 || bits > pqi::kMaxBits) return PQ_EINVAL;
  const Codebook& cb = codebook(bits);
  if (centroids) std::copy(cb.c.begin(), cb.c.end(), centroids);
  if (boundaries) std::copy(cb.beta.begin(), cb.beta.end(), boundaries);
  if (mse) *mse = cb.mse;
  return PQ_OK;
}


int pq_quantize(int d, int bits, int in_dtype, const void* x, int64_t n_blocks, const uint8_t* signs,
                int m, const uint16_t* proj, uint8_t* codes, uint16_t* norms, uint8_t* qjl_bits,
                uint16_t* rnorms, void* stream) {
  return quantize_impl(d, bits, in_dtype, x, n_blocks, signs, m, proj, codes, norms, qjl_bits, rnorms, 0, stream);
}

int pq_dequantize(int d, int bits, const uint8_t* codes, const uint16_t* norms, int64_t n_blocks,
                  const uint8_t* signs, int out_dtype, void* out, void* stream) {
  return dequantize_impl(d, bits, codes, norms, n_blocks, signs, out_dtype, out, 0, stream);
}

int pq_quantize_packed(int d, int bits, int in_dtype, const void* x, int64_t n_blocks, const uint8_t* signs,
                       int m, const uint16_t* proj, uint8_t* codes, uint16_t* norms, uint8_t* qjl_bits,
                       uint16_t* rnorms, void* stream) {
  if (bits < 1 || bits > pqi::kMaxBits) return PQ_EINVAL;
  // at 8 bits the stream is one byte per code
  return quantize_impl(d, bits, in_dtype, x, n_blocks, signs, m, proj, codes, norms, qjl_bits, rnorms,
                       bits == 8 ? 0 : bits, stream);
}

int pq_dequantize_packed(int d, int bits, const uint8_t* codes, const uint16_t* norms, int64_t n_blocks,
                         const uint8_t* signs, int out_dtype, void* out, void* stream) {
  if (bits < 1 || bits > pqi::kMaxBits) return PQ_EINVAL;
  return dequantize_impl(d, bits, codes, norms, n_blocks, signs, out_dtype, out, bits == 8 ? 0 : bits, stream);
}

int pq_quantize_many(int d, int bits, int in_dtype, int packed, int n_tensors, const pq_tensor* table, void* stream) {
  int st = check_d(d);
  if (st) return st;
  if (bits < 1 || bits > pqi::kMaxBits) return PQ_EINVAL;
  if (in_dtype != PQ_F32 && in_dtype != PQ_BF16) return PQ_EINVAL;
  if (packed != 0 && packed != 1) return PQ_EINVAL;
  if (n_tensors < 0) return PQ_EINVAL;
  if (n_tensors == 0) return PQ_OK;
  if (!table || !aligned(table, 8)) return PQ_EINVAL;
  pqi::LaunchCfg cfg;
  if ((st = launch_cfg(&cfg))) return st;
  pqi::QuantArgs a;
  std::memset(&a, 0, sizeof(a));
  a.pbits = packed && bits < 8 ? bits : 0;                         // 8 bits packed is the byte layout
  a.t = make_tables(bits);
  return hip_status(pqi::launch_quantize_many(d, in_dtype == PQ_BF16, a, table, n_tensors, cfg, (hipStream_t)stream));
}

int pq_dequantize_many(int d, int bits, int out_dtype, int packed, int n_tensors, const pq_tensor* table,
                       void* stream) {
  int st = check_d(d);
  if (st) return st;
  if (bits < 1 || bits > pqi::kMaxBits) return PQ_EINVAL;
  if (out_dtype != PQ_F32 && out_dtype != PQ_BF16) return PQ_EINVAL;
  if (packed != 0 && packed != 1) return PQ_EINVAL;
  if (n_tensors < 0) return PQ_EINVAL;
  if (n_tensors == 0) return PQ_OK;
  if (!table || !aligned(table, 8)) return PQ_EINVAL;
  pqi::LaunchCfg cfg;
  if ((st = launch_cfg(&cfg))) return st;
  pqi::DequantArgs a;
  std::memset(&a, 0, sizeof(a));
  a.pbits = packed && bits < 8 ? bits : 0;                         // 8 bits packed is the byte layout
  a.t = make_tables(bits);
  return hip_status(pqi::launch_dequantize_many(d, out_dtype == PQ_BF16, a, table, n_tensors, cfg, (hipStream_t)stream));
}

int qjl_sketch(int d, int m, const uint16_t* keys, int64_t n_keys, const uint16_t* proj, uint8_t* bits,
               uint16_t* norms, void* stream) {
  int st = check_d(d);
  if (st) return st;
  if (m <= 0 || (m % 8) != 0) return PQ_EINVAL;
  if (m > 1024) return PQ_EUNSUPPORTED;
  if (n_keys < 0 || n_keys > kMaxElems / d) return PQ_EINVAL;
  if (n_keys == 0) return PQ_OK;
  if (!keys || !proj || !bits || !norms) return PQ_EINVAL;
  if (!aligned(keys, 16) || !aligned(proj, 16) || !aligned(bits, 16) || !aligned(norms, 2)) return PQ_EINVAL;
  pqi::LaunchCfg cfg;
  if ((st = launch_cfg(&cfg))) return st;
  pqi::SketchArgs a;
  std::memset(&a, 0, sizeof(a));
  a.keys = keys; a.n_keys = n_keys; a.proj = proj; a.bits = bits; a.norms = norms; a.m = m;
  return hip_status(pqi::launch_sketch(d, a, cfg, (hipStream_t)stream));
}

int qjl_outlier_channels(int d, const uint16_t* keys, int64_t n_heads, int64_t seq_len, int group_size, int n_out,
                         uint8_t* idx, void* stream) {
  int st = check_d(d);
  if (st) return st;
  if (d > 256) return PQ_EUNSUPPORTED;                    // channel indices are bytes
  if (n_heads < 0 || seq_len < 0 || group_size < 1 || n_out < 1 || n_out > d) return PQ_EINVAL;
  if (n_heads > 0 && seq_len > kMaxElems / d / n_heads) return PQ_EINVAL;
  if (n_heads == 0 || seq_len == 0) return PQ_OK;
  if (!keys || !idx) return PQ_EINVAL;
  if (!aligned(keys, 16)) return PQ_EINVAL;
  pqi::OutlierArgs a;
  a.keys = keys; a.n_heads = n_heads; a.seq_len = seq_len; a.n_groups = (seq_len + group_size - 1) / group_size;
  a.d = d; a.group_size = group_size; a.n_out = n_out; a.oidx = idx;
  return hip_status(pqi::launch_outliers(a, (hipStream_t)stream));
}

int qjl_sketch_split(int d, int m, const uint16_t* keys, int64_t n_heads, int64_t seq_len, int group_size,
                     int n_out, const uint8_t* idx, int part, const uint16_t* proj, uint8_t* bits, uint16_t* norms,
                     void* stream) {
  int st = check_d(d);
  if (st) return st;
  if (d > 256) return PQ_EUNSUPPORTED;
  if (m <= 0 || (m % 8) != 0) return PQ_EINVAL;
  if (m > 1024) return PQ_EUNSUPPORTED;
  if (n_heads < 0 || seq_len < 0 || group_size < 1 || n_out < 1 || n_out > d || (part != 0 && part != 1))
    return PQ_EINVAL;
  if (n_heads > 0 && seq_len > kMaxElems / d / n_heads) return PQ_EINVAL;
  if (n_heads == 0 || seq_len == 0) return PQ_OK;
  if (!keys || !idx || !proj || !bits || !norms) return PQ_EINVAL;
  if (!aligned(keys, 16) || !aligned(proj, 16) || !aligned(bits, 16) || !aligned(norms, 2)) return PQ_EINVAL;
  pqi::LaunchCfg cfg;
  if ((st = launch_cfg(&cfg))) return st;
  pqi::SketchArgs a;
  a.keys = keys; a.n_keys = n_heads * seq_len; a.proj = proj; a.bits = bits; a.norms = norms; a.m = m;
  a.oidx = idx; a.seq_len = seq_len; a.n_groups = (seq_len + group_size - 1) / group_size;
  a.group_size = group_size; a.n_out = n_out; a.part = part;
  return hip_status(pqi::launch_sketch(d, a, cfg, (hipStream_t)stream));
}

int qjl_project(int d, int m, const uint16_t* q, int64_t n_q, const uint16_t* proj, float* sq,
                void* stream) {
  int st = check_d(d);
  if (st) return st;
  if (m <= 0 || (m % 8) != 0) return PQ_EINVAL;
  if (m > 1024) return PQ_EUNSUPPORTED;
  if (n_q < 0 || n_q > (int64_t)INT32_MAX / m) return PQ_EINVAL;
  if (n_q == 0) return PQ_OK;
  if (!q || !proj || !sq) return PQ_EINVAL;
  if (!aligned(q, 16) || !aligned(proj, 16) || !aligned(sq, 4)) return PQ_EINVAL;
  pqi::ProjectArgs a;
  a.q = q; a.n_q = n_q; a.proj = proj; a.sq = sq; a.d = d; a.m = m;
  a.rows_per_group = n_q; a.group_stride = n_q * m;
  return hip_status(pqi::launch_project(a, (hipStream_t)stream));
}

static int score_qjl_impl(int m, int batch, int kv_heads, int q_heads, int64_t n_keys, const float* sq,
                          const uint8_t* bits, const uint16_t* norms, float* scores, int accumulate, void* stream) {
  if (m <= 0 || (m % 8) != 0) return PQ_EINVAL;
  if ((m % 64) != 0 || m > 1024) return PQ_EUNSUPPORTED;
  if (batch < 0 || kv_heads <= 0 || q_heads <= 0 || n_keys < 0) return PQ_EINVAL;
  if (q_heads % kv_heads != 0) return PQ_EINVAL;
  if (q_heads / kv_heads > 4) return PQ_EUNSUPPORTED;
  if ((int64_t)batch * kv_heads > INT32_MAX / 1024) return PQ_EINVAL;
  if (n_keys > kMaxElems / ((int64_t)batch * q_heads + 1)) return PQ_EINVAL;
  if (batch == 0 || n_keys == 0) return PQ_OK;
  if (!sq || !bits || !norms || !scores) return PQ_EINVAL;
  if (!aligned(sq, 4) || !aligned(bits, 16) || !aligned(scores, 4) || !aligned(norms, 2)) return PQ_EINVAL;
  pqi::LaunchCfg cfg;
  int st2 = launch_cfg(&cfg);
  if (st2) return st2;
  pqi::ScoreArgs a;
  a.sq = sq; a.bits = bits; a.norms = norms; a.scores = scores; a.n_keys = n_keys; a.m = m;
  a.batch = batch; a.kv_heads = kv_heads; a.q_heads = q_heads; a.accumulate = accumulate;
  return hip_status(pqi::launch_score(a, cfg, (hipStream_t)stream));
}

int qjl_score(int m, int batch, int kv_heads, int q_heads, int64_t n_keys, const float* sq,
              const uint8_t* bits, const uint16_t* norms, float* scores, void* stream) {
  return score_qjl_impl(m, batch, kv_heads, q_heads, n_keys, sq, bits, norms, scores, 0, stream);
}

int qjl_score_add(int m, int batch, int kv_heads, int q_heads, int64_t n_keys, const float* sq,
                  const uint8_t* bits, const uint16_t* norms, float* scores, void* stream) {
  return score_qjl_impl(m, batch, kv_heads, q_heads, n_keys, sq, bits, norms, scores, 1, stream);
}

int64_t pq_query_prep_bytes(int d, int m, int n_heads) {
  if (check_d(d) || m < 0 || (m % 64) != 0 || m > 1024 || n_heads < 0) return -1;
  return (int64_t)n_heads * pqi::prep_head_bytes(d, m);
}

int pq_query_prep(int d, int m, int n_heads, int n_q, const uint16_t* q, const uint8_t* signs,
                  const uint16_t* proj, void* prep, void* stream) {
  int st = check_d(d);
  if (st) return st;
  if (m < 0 || (m % 8) != 0) return PQ_EINVAL;
  if ((m % 64) != 0 || m > 1024) return PQ_EUNSUPPORTED;
  if (n_heads < 0 || n_q < 0 || n_q > pqi::kScoreRows) return PQ_EINVAL;
  if (n_heads > INT32_MAX / pqi::kScoreRows) return PQ_EINVAL;
  if (m == 0 && proj) return PQ_EINVAL;
  if (n_heads == 0) return PQ_OK;
  if (!signs || !prep || (n_q > 0 && !q) || (m > 0 && !proj)) return PQ_EINVAL;
  if (!aligned(prep, 16) || (q && !aligned(q, 16)) || (proj && !aligned(proj, 16))) return PQ_EINVAL;
  pqi::QueryPrepArgs a;
  a.q = q; a.signs = signs; a.proj = proj; a.prep = static_cast<unsigned char*>(prep);
  a.n_heads = n_heads; a.n_q = n_q; a.d = d; a.m = m;
  return hip_status(pqi::launch_query_prep(a, (hipStream_t)stream));
}

static int score_impl(int d, int bits, int m, int n_heads, int n_q, int64_t n_tok, const void* prep,
                      const uint8_t* codes, const uint16_t* norms, const uint8_t* qjl_bits, const uint16_t* rnorms,
                      float* scores, int packed, void* stream) {
  int st = check_d(d);
  if (st) return st;
  if (bits < 1 || bits > pqi::kMaxBits) return PQ_EINVAL;
  if (bits > pqi::kMaxScoreBits) return PQ_EUNSUPPORTED;
  if (m < 0 || (m % 8) != 0) return PQ_EINVAL;
  if ((m % 64) != 0 || m > 1024) return PQ_EUNSUPPORTED;
  if (pqi::prep_head_bytes(d, m) - pqi::prep_off_meta(d, m) > 65536) return PQ_EUNSUPPORTED;
  if (n_heads < 0 || n_q < 0 || n_q > pqi::kScoreRows || n_tok < 0) return PQ_EINVAL;
  if (n_tok > kMaxElems / ((int64_t)d * (n_heads + 1))) return PQ_EINVAL;
  if (m == 0 && (qjl_bits || rnorms)) return PQ_EINVAL;
  if (n_heads == 0 || n_q == 0 || n_tok == 0) return PQ_OK;
  if (!prep || !codes || !norms || !scores) return PQ_EINVAL;
  if (m > 0 && (!qjl_bits || !rnorms)) return PQ_EINVAL;
  if (!aligned(prep, 16) || !aligned(codes, 16) || !aligned(norms, 2) || !aligned(scores, 4)) return PQ_EINVAL;
  if (m > 0 && (!aligned(qjl_bits, 2) || !aligned(rnorms, 2))) return PQ_EINVAL;
  pqi::LaunchCfg cfg;
  if ((st = launch_cfg(&cfg))) return st;
  pqi::TwoStageArgs a;
  std::memset(&a, 0, sizeof(a));
  a.prep = static_cast<const unsigned char*>(prep);
  a.codes = codes; a.norms = norms; a.qbits = qjl_bits; a.rnorms = rnorms; a.scores = scores;
  a.n_tok = n_tok; a.n_heads = n_heads; a.n_q = n_q; a.m = m; a.packed = packed;
  // Walsh coefficients of the codebook over the odd subsets of the code bits:
  // alpha_p = 2^-b sum_k c_k s_p(k); the even subsets vanish by antisymmetry
  const Codebook& cb = codebook(bits);
  const int L = 1 << bits;
  for (int p = 0; p < (L >> 1); ++p) {
    const uint32_t mask = pqi::plane_mask(bits, p);
    double acc = 0.0;
    for (int k = 0; k < L; ++k) acc += (__builtin_popcount((uint32_t)k & mask) & 1) ? cb.c[k] : -cb.c[k];
    a.alpha[p] = acc / (double)L;
  }
  return hip_status(pqi::launch_two_stage(d, bits, a, cfg, (hipStream_t)stream));
}

int pq_score(int d, int bits, int m, int n_heads, int n_q, int64_t n_tok, const void* prep,
             const uint8_t* codes, const uint16_t* norms, const uint8_t* qjl_bits, const uint16_t* rnorms,
             float* scores, void* stream) {
  return score_impl(d, bits, m, n_heads, n_q, n_tok, prep, codes, norms, qjl_bits, rnorms, scores, 0, stream);
}

int pq_score_packed(int d, int bits, int m, int n_heads, int n_q, int64_t n_tok, const void* prep,
                    const uint8_t* codes, const uint16_t* norms, const uint8_t* qjl_bits, const uint16_t* rnorms,
                    float* scores, void* stream) {
  return score_impl(d, bits, m, n_heads, n_q, n_tok, prep, codes, norms, qjl_bits, rnorms, scores, 1, stream);
}

int64_t pq_attention_work_bytes(int d, int n_heads, int64_t n_tok) {
  if (check_d(d) || n_heads < 0 || n_heads > INT32_MAX / pqi::kScoreRows || n_tok < 0) return -1;
  if (n_tok > kMaxElems / ((int64_t)d * (n_heads + 1))) return -1;
  return pqi::attn_work_bytes(d, n_heads, n_tok);
}

// Work buffer of pq_attention_noalloc: a fixed array in device memory (one copy per device, at
// its own address on each), used by every call on that device.  Host code never passes the
// array's name to a kernel: it reads the array's device address once per device with
// hipGetSymbolAddress, with that device current, and passes that address.
static constexpr int64_t kAttnScratchBytes = (int64_t)PQ_ATTN_NOALLOC_MAX_WORK;
static __device__ __align__(256) unsigned char scratch[kAttnScratchBytes];

static constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's copy of `scratch`, looked up on the first call per device.
static int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return PQ_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (!p) return PQ_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PQ_OK;
}

// work == nullptr with use_scratch: the work buffer is this device's `scratch` array, fetched
// after every argument has been validated.
static int attention_impl(int d, int bits, int m, int n_heads, int n_q, int64_t n_tok, const void* prep,
                          const uint8_t* k_codes, const uint16_t* k_norms, const uint8_t* k_qjl_bits,
                          const uint16_t* k_rnorms, const uint8_t* v_codes, const uint16_t* v_norms,
                          const uint8_t* v_signs, int64_t n_win, const uint16_t* k_win, const uint16_t* v_win,
                          const uint16_t* q, float sm_scale, void* work, float* out, int packed, void* stream,
                          bool use_scratch = false) {
  int st = check_d(d);
  if (st) return st;
  if (bits < 1 || bits > pqi::kMaxBits) return PQ_EINVAL;
  if (bits > pqi::kMaxScoreBits) return PQ_EUNSUPPORTED;
  if (m < 0 || (m % 8) != 0) return PQ_EINVAL;
  if ((m % 64) != 0 || m > 1024) return PQ_EUNSUPPORTED;
  if (pqi::prep_head_bytes(d, m) - pqi::prep_off_meta(d, m) > 65536) return PQ_EUNSUPPORTED;
  if (n_heads < 0 || n_heads > INT32_MAX / pqi::kScoreRows || n_q < 0 || n_q > pqi::kScoreRows) return PQ_EINVAL;
  if (n_tok < 0 || n_win < 0) return PQ_EINVAL;
  if (n_tok > kMaxElems / ((int64_t)d * (n_heads + 1))) return PQ_EINVAL;
  if (n_win > pqi::kAttnMaxWin) return PQ_EUNSUPPORTED;
  if (!std::isfinite(sm_scale)) return PQ_EINVAL;
  if (m == 0 && (k_qjl_bits || k_rnorms)) return PQ_EINVAL;
  if (n_heads == 0 || n_q == 0) return PQ_OK;
  if (n_tok + n_win == 0) return PQ_EINVAL;             // softmax over no token
  if (!v_signs || !out) return PQ_EINVAL;
  if (n_tok > 0) {
    if (!prep || !k_codes || !k_norms || !v_codes || !v_norms || (!work && !use_scratch)) return PQ_EINVAL;
    if (m > 0 && (!k_qjl_bits || !k_rnorms)) return PQ_EINVAL;
    if (!aligned(prep, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) || !aligned(k_norms, 2) ||
        !aligned(v_norms, 2) || (!use_scratch && !aligned(work, 16)))
      return PQ_EINVAL;
    if (m > 0 && (!aligned(k_qjl_bits, 2) || !aligned(k_rnorms, 2))) return PQ_EINVAL;
  }
  if (n_win > 0 && (!k_win || !v_win || !q || !aligned(k_win, 16) || !aligned(v_win, 16) || !aligned(q, 2)))
    return PQ_EINVAL;
  if (!aligned(out, 4)) return PQ_EINVAL;
  if (use_scratch && n_tok > 0) {
    if (pqi::attn_work_bytes(d, n_heads, n_tok) > kAttnScratchBytes) return PQ_ETOOBIG;
    if ((st = scratch_address(&work))) return st;
  }
  const pqi::AttnPlan plan = pqi::attn_plan(d, n_heads, n_tok);
  pqi::AttnArgs a;
  std::memset(&a, 0, sizeof(a));
  a.prep = static_cast<const unsigned char*>(prep);
  a.k_codes = k_codes; a.k_norms = k_norms; a.k_qbits = k_qjl_bits; a.k_rnorms = k_rnorms;
  a.v_codes = v_codes; a.v_norms = v_norms; a.v_signs = v_signs;
  a.k_win = k_win; a.v_win = v_win; a.q = q; a.out = out;
  a.work_ml = static_cast<float*>(work);
  a.work_o = plan.n_parts ? a.work_ml + (int64_t)n_heads * plan.n_parts * pqi::kScoreRows * 2 : nullptr;
  a.n_tok = n_tok; a.n_win = n_win; a.tiles_per_range = plan.tiles_per_range;
  a.n_heads = n_heads; a.n_q = n_q; a.m = m; a.n_ranges = plan.n_ranges; a.n_parts = plan.n_parts;
  a.packed = packed;
  a.scale_log2 = (double)sm_scale * 1.4426950408889634;          // log2(e)
  const Codebook& cb = codebook(bits);
  const int L = 1 << bits;
  for (int p = 0; p < (L >> 1); ++p) {
    const uint32_t mask = pqi::plane_mask(bits, p);
    double acc = 0.0;
    for (int k = 0; k < L; ++k) acc += (__builtin_popcount((uint32_t)k & mask) & 1) ? cb.c[k] : -cb.c[k];
    a.alpha[p] = acc / (double)L;
  }
  for (int k = 0; k < L; ++k) a.vcent[k] = (float)cb.c[k];
  return hip_status(pqi::launch_attention(d, bits, a, (hipStream_t)stream));
}

int pq_attention(int d, int bits, int m, int n_heads, int n_q, int64_t n_tok, const void* prep,
                 const uint8_t* k_codes, const uint16_t* k_norms, const uint8_t* k_qjl_bits, const uint16_t* k_rnorms,
                 const uint8_t* v_codes, const uint16_t* v_norms, const uint8_t* v_signs, int64_t n_win,
                 const uint16_t* k_win, const uint16_t* v_win, const uint16_t* q, float sm_scale, void* work,
                 float* out, void* stream) {
  return attention_impl(d, bits, m, n_heads, n_q, n_tok, prep, k_codes, k_norms, k_qjl_bits, k_rnorms, v_codes,
                        v_norms, v_signs, n_win, k_win, v_win, q, sm_scale, work, out, 0, stream);
}

int pq_attention_packed(int d, int bits, int m, int n_heads, int n_q, int64_t n_tok, const void* prep,
                        const uint8_t* k_codes, const uint16_t* k_norms, const uint8_t* k_qjl_bits,
                        const uint16_t* k_rnorms, const uint8_t* v_codes, const uint16_t* v_norms,
                        const uint8_t* v_signs, int64_t n_win, const uint16_t* k_win, const uint16_t* v_win,
                        const uint16_t* q, float sm_scale, void* work, float* out, void* stream) {
  return attention_impl(d, bits, m, n_heads, n_q, n_tok, prep, k_codes, k_norms, k_qjl_bits, k_rnorms, v_codes,
                        v_norms, v_signs, n_win, k_win, v_win, q, sm_scale, work, out, 1, stream);
}

int pq_probe_stream(const uint8_t* in, uint16_t* out, int64_t n, void* stream) {
  if (n < 0 || n > kMaxElems) return PQ_EINVAL;
  if (n == 0) return PQ_OK;
  if (!in || !out || !aligned(in, 16) || !aligned(out, 16)) return PQ_EINVAL;
  pqi::LaunchCfg cfg;
  int st = launch_cfg(&cfg);
  if (st) return st;
  return hip_status(pqi::launch_stream_probe(in, out, n, cfg, (hipStream_t)stream));
}

int pq_attention_noalloc(int d, int bits, int m, int n_heads, int n_q, int64_t n_tok, const void* prep,
                         const uint8_t* k_codes, const uint16_t* k_norms, const uint8_t* k_qjl_bits,
                         const uint16_t* k_rnorms, const uint8_t* v_codes, const uint16_t* v_norms,
                         const uint8_t* v_signs, int64_t n_win, const uint16_t* k_win, const uint16_t* v_win,
                         const uint16_t* q, float sm_scale, int packed, float* out, void* stream) {
  if (packed != 0 && packed != 1) return PQ_EINVAL;
  return attention_impl(d, bits, m, n_heads, n_q, n_tok, prep, k_codes, k_norms, k_qjl_bits, k_rnorms, v_codes,
                        v_norms, v_signs, n_win, k_win, v_win, q, sm_scale, nullptr, out, packed, stream, true);
}

int pq_quantize_bd(int d, int bits, int in_dtype, const void* x, int64_t n_blocks, const uint8_t* signs,
                   uint8_t* codes, uint16_t* norms, void* stream) {
  int st = check_d_bd(d);
  if (st) return st;
  if (bits < 1 || bits > pqi::kMaxBits) return PQ_EINVAL;
  if (in_dtype != PQ_F32 && in_dtype != PQ_BF16) return PQ_EINVAL;
  if (n_blocks < 0 || n_blocks > kMaxElems / d) return PQ_EINVAL;
  if (n_blocks == 0) return PQ_OK;
  if (!x || !signs || !codes || !norms) return PQ_EINVAL;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(norms, 2)) return PQ_EINVAL;
  pqi::LaunchCfg cfg;
  if ((st = launch_cfg(&cfg))) return st;
  pqi::BdArgs a;
  std::memset(&a, 0, sizeof(a));
  a.x = x; a.codes = codes; a.norms = norms; a.signs = signs; a.n_blocks = n_blocks; a.d = d; a.bits = bits;
  fill_bd_codebook(bits, a);
  return hip_status(pqi::launch_quantize_bd(in_dtype == PQ_BF16, a, cfg, (hipStream_t)stream));
}

int pq_dequantize_bd(int d, int bits, const uint8_t* codes, const uint16_t* norms, int64_t n_blocks,
                     const uint8_t* signs, int out_dtype, void* out, void* stream) {
  int st = check_d_bd(d);
  if (st) return st;
  if (bits < 1 || bits > pqi::kMaxBits) return PQ_EINVAL;
  if (out_dtype != PQ_F32 && out_dtype != PQ_BF16) return PQ_EINVAL;
  if (n_blocks < 0 || n_blocks > kMaxElems / d) return PQ_EINVAL;
  if (n_blocks == 0) return PQ_OK;
  if (!codes || !norms || !signs || !out) return PQ_EINVAL;
  if (!aligned(codes, 16) || !aligned(out, 16) || !aligned(norms, 2)) return PQ_EINVAL;
  pqi::LaunchCfg cfg;
  if ((st = launch_cfg(&cfg))) return st;
  pqi::BdArgs a;
  std::memset(&a, 0, sizeof(a));
  a.ccodes = codes; a.cnorms = norms; a.signs = signs; a.out = out; a.n_blocks = n_blocks; a.d = d; a.bits = bits;
  fill_bd_codebook(bits, a);
  return hip_status(pqi::launch_dequantize_bd(out_dtype == PQ_BF16, a, cfg, (hipStream_t)stream));
}

int pq_quantize_dense(int d, int bits, int in_dtype, const void* x, int64_t n_blocks, const float* rot,
                      uint8_t* codes, uint16_t* norms, void* stream) {
  int st = check_d_dense(d);
  if (st) return st;
  if (bits < 1 || bits > pqi::kMaxBits) return PQ_EINVAL;
  if (in_dtype != PQ_F32 && in_dtype != PQ_BF16) return PQ_EINVAL;
  if (n_blocks < 0 || n_blocks > kMaxElems / d) return PQ_EINVAL;
  if (n_blocks == 0) return PQ_OK;
  if (!x || !rot || !codes || !norms) return PQ_EINVAL;
  if (!aligned(x, 4) || !aligned(rot, 4) || !aligned(norms, 2)) return PQ_EINVAL;
  pqi::LaunchCfg cfg;
  if ((st = launch_cfg(&cfg))) return st;
  pqi::BdArgs a;
  std::memset(&a, 0, sizeof(a));
  a.x = x; a.codes = codes; a.norms = norms; a.rot = rot; a.n_blocks = n_blocks; a.d = d; a.bits = bits;
  const Codebook& cb = sphere_codebook(bits, d);
  for (int k = 0; k < (1 << bits); ++k) a.cent[k] = (float)cb.c[k];
  for (int k = 0; k + 1 < (1 << bits); ++k) {
    a.beta[k] = (float)cb.beta[k];
    a.beta_lo[k] = (float)(cb.beta[k] - (double)a.beta[k]);
  }
  // search grid of the matrix-core kernel: cells 0.9 of the smallest boundary gap wide over
  // [-(max |beta| + w), max |beta| + w] (at most 4096 cells, else the kernel bisects)
  {
    const int nb = (1 << bits) - 1;
    double gap = INFINITY, top = 0.0;
    for (int k = 0; k + 1 < nb; ++k) gap = std::min(gap, (double)a.beta[k + 1] - (double)a.beta[k]);
    for (int k = 0; k < nb; ++k) top = std::max(top, std::fabs((double)a.beta[k]));
    const double w = nb == 1 ? 0.5 : 0.9 * gap;
    const int half = (int)std::ceil((top + w) / w);
    if (w > 0.0 && 2 * half + 1 <= 4096) {
      a.half = half;
      a.ncell = 2 * half + 1;
      a.cell_w = (float)w;
      a.cell_inv_w = (float)(1.0 / w);
    }
  }
  return hip_status(pqi::launch_quantize_dense(in_dtype == PQ_BF16, a, cfg, (hipStream_t)stream));
}

int pq_dequantize_dense(int d, int bits, const uint8_t* codes, const uint16_t* norms, int64_t n_blocks,
                        const float* rot, int out_dtype, void* out, void* stream) {
  int st = check_d_dense(d);
  if (st) return st;
  if (bits < 1 || bits > pqi::kMaxBits) return PQ_EINVAL;
  if (out_dtype != PQ_F32 && out_dtype != PQ_BF16) return PQ_EINVAL;
  if (n_blocks < 0 || n_blocks > kMaxElems / d) return PQ_EINVAL;
  if (n_blocks == 0) return PQ_OK;
  if (!codes || !norms || !rot || !out) return PQ_EINVAL;
  if (!aligned(codes, 16) || !aligned(out, 4) || !aligned(rot, 4) || !aligned(norms, 2)) return PQ_EINVAL;
  pqi::LaunchCfg cfg;
  if ((st = launch_cfg(&cfg))) return st;
  pqi::BdArgs a;
  std::memset(&a, 0, sizeof(a));
  a.ccodes = codes; a.cnorms = norms; a.rot = rot; a.out = out; a.n_blocks = n_blocks; a.d = d; a.bits = bits;
  const Codebook& cb = sphere_codebook(bits, d);
  for (int k = 0; k < (1 << bits); ++k) a.cent[k] = (float)cb.c[k];
  return hip_status(pqi::launch_dequantize_dense(out_dtype == PQ_BF16, a, cfg, (hipStream_t)stream));
}

int pq_sphere_codebook(int bits, int d, double* centroids, double* boundaries) {
  if (bits < 1 || bits > pqi::kMaxBits || d < 3) return PQ_EINVAL;
  const Codebook& cb = sphere_codebook(bits, d);
  if (centroids) for (int k = 0; k < (1 << bits); ++k) centroids[k] = cb.c[k];
  if (boundaries) for (int k = 0; k + 1 < (1 << bits); ++k) boundaries[k] = cb.beta[k];
  return PQ_OK;
}

}  // extern "C"
