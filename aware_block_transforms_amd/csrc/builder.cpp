// Host-side (CPU, fp64) part of libwush: status strings, the thread-local
// error text, block second moments and the per-block transform builder.
//
// The builder follows the WUSH news article (chain.bitekongjian.com),
// paragraph on the construction (Cholesky factor of weight statistics, U and S
// of an SVD, a Hadamard matrix; non-orthogonal, block-diagonal) and paragraph
// on deployment (second moments from calibration data, per-block Cholesky and
// SVD that can run in parallel).  The SVD factors are those of
// K = W'^T X_b / sqrt(n); they are obtained from the symmetric
// eigen-decomposition of C = K K^T = W'^T Sx_b W' with a cyclic Jacobi
// method, which is accurate to a few ulps for these small (16x16, 32x32)
// matrices.  Blocks are independent and are spread over std::threads.

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "common.h"

namespace wush {

static thread_local std::string g_last_error;

wush_status fail(wush_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

namespace {

// Run fn(b) for b in [0, count) on up to hardware_concurrency threads.
template <class F>
void parallel_blocks(int count, F fn) {
  unsigned hw = std::max(1u, std::thread::hardware_concurrency());
  int nth = static_cast<int>(std::min<unsigned>(hw, static_cast<unsigned>(count)));
  if (nth <= 1) {
    for (int b = 0; b < count; ++b) fn(b);
    return;
  }
  std::atomic<int> next{0};
  std::vector<std::thread> pool;
  for (int t = 0; t < nth; ++t)
    pool.emplace_back([&] {
      for (int b = next++; b < count; b = next++) fn(b);
    });
  for (auto& th : pool) th.join();
}

// In-place lower Cholesky of the bs x bs matrix a (row-major).  Returns false
// when a pivot is not positive.
bool cholesky_lower(double* a, int bs) {
  for (int j = 0; j < bs; ++j) {
    double d = a[j * bs + j];
    for (int k = 0; k < j; ++k) d -= a[j * bs + k] * a[j * bs + k];
    if (!(d > 0.0)) return false;
    double ljj = std::sqrt(d);
    a[j * bs + j] = ljj;
    for (int i = j + 1; i < bs; ++i) {
      double s = a[i * bs + j];
      for (int k = 0; k < j; ++k) s -= a[i * bs + k] * a[j * bs + k];
      a[i * bs + j] = s / ljj;
    }
    for (int k = j + 1; k < bs; ++k) a[j * bs + k] = 0.0;
  }
  return true;
}

// Cyclic Jacobi eigen-decomposition of the symmetric matrix a (destroyed).
// On return lam[i] are the eigenvalues and column i of v (row-major,
// v[r*bs+i]) the matching unit eigenvector.
void jacobi_eigh(double* a, int bs, double* lam, double* v) {
  for (int i = 0; i < bs * bs; ++i) v[i] = 0.0;
  for (int i = 0; i < bs; ++i) v[i * bs + i] = 1.0;
  for (int sweep = 0; sweep < 100; ++sweep) {
    double off = 0.0, diag = 0.0;
    for (int p = 0; p < bs; ++p) {
      diag += a[p * bs + p] * a[p * bs + p];
      for (int q = p + 1; q < bs; ++q) off += a[p * bs + q] * a[p * bs + q];
    }
    if (off <= 1e-34 * diag || off == 0.0) break;
    for (int p = 0; p < bs - 1; ++p) {
      for (int q = p + 1; q < bs; ++q) {
        double apq = a[p * bs + q];
        if (apq == 0.0) continue;
        double app = a[p * bs + p], aqq = a[q * bs + q];
        double theta = (aqq - app) / (2.0 * apq);
        double t = (theta >= 0 ? 1.0 : -1.0) / (std::fabs(theta) + std::sqrt(theta * theta + 1.0));
        double c = 1.0 / std::sqrt(t * t + 1.0);
        double s = t * c;
        // A <- J^T A J with J the rotation in the (p, q) plane
        for (int k = 0; k < bs; ++k) {
          double akp = a[k * bs + p], akq = a[k * bs + q];
          a[k * bs + p] = c * akp - s * akq;
          a[k * bs + q] = s * akp + c * akq;
        }
        for (int k = 0; k < bs; ++k) {
          double apk = a[p * bs + k], aqk = a[q * bs + k];
          a[p * bs + k] = c * apk - s * aqk;
          a[q * bs + k] = s * apk + c * aqk;
        }
        a[p * bs + q] = a[q * bs + p] = 0.0;
        for (int k = 0; k < bs; ++k) {
          double vkp = v[k * bs + p], vkq = v[k * bs + q];
          v[k * bs + p] = c * vkp - s * vkq;
          v[k * bs + q] = s * vkp + c * vkq;
        }
      }
    }
  }
  for (int i = 0; i < bs; ++i) lam[i] = a[i * bs + i];
}

// Entry (i, j) of the orthonormal Sylvester Hadamard matrix of order bs.
inline double hadamard_entry(int i, int j, int bs) {
  return (__builtin_popcount(static_cast<unsigned>(i & j)) & 1 ? -1.0 : 1.0) / std::sqrt(double(bs));
}

const double kDamping[] = {0.0, 1e-10, 1e-8, 1e-6, 1e-4, 1e-2};

// Build T_X and T_W (fp64, bs x bs, row-major) for one block from its weight
// moment A and activation moment B.  Returns false if no rung of the damping
// ladder yields a Cholesky factor.
bool block_transform(bool with_h, int bs, const double* A, const double* B, double* tx, double* tw) {
  std::vector<double> L(bs * bs), C(bs * bs), tmp(bs * bs), U(bs * bs), lam(bs), Linv(bs * bs);
  double tr = 0.0;
  for (int i = 0; i < bs; ++i) tr += A[i * bs + i];
  bool ok = false;
  for (double eps : kDamping) {
    for (int i = 0; i < bs * bs; ++i) L[i] = A[i];
    for (int i = 0; i < bs; ++i) L[i * bs + i] += eps * (tr / bs);
    if (cholesky_lower(L.data(), bs)) { ok = true; break; }
  }
  if (!ok) return false;
  // C = L^T B L  (symmetrised)
  for (int i = 0; i < bs; ++i)
    for (int j = 0; j < bs; ++j) {
      double s = 0.0;
      for (int k = 0; k < bs; ++k) s += B[i * bs + k] * L[k * bs + j];
      tmp[i * bs + j] = s;                     // B L
    }
  for (int i = 0; i < bs; ++i)
    for (int j = 0; j < bs; ++j) {
      double s = 0.0;
      for (int k = 0; k < bs; ++k) s += L[k * bs + i] * tmp[k * bs + j];
      C[i * bs + j] = s;
    }
  for (int i = 0; i < bs; ++i)
    for (int j = i + 1; j < bs; ++j) {
      double m = 0.5 * (C[i * bs + j] + C[j * bs + i]);
      C[i * bs + j] = C[j * bs + i] = m;
    }
  std::vector<double> V(bs * bs);
  jacobi_eigh(C.data(), bs, lam.data(), V.data());
  // sort descending (stable), sign rule: largest-|.| entry of each column positive
  std::vector<int> order(bs);
  for (int i = 0; i < bs; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return lam[x] > lam[y]; });
  std::vector<double> sig(bs);
  for (int c = 0; c < bs; ++c) {
    int src = order[c];
    int piv = 0;
    for (int r = 1; r < bs; ++r)
      if (std::fabs(V[r * bs + src]) > std::fabs(V[piv * bs + src])) piv = r;
    double sg = V[piv * bs + src] < 0 ? -1.0 : 1.0;
    for (int r = 0; r < bs; ++r) U[r * bs + c] = sg * V[r * bs + src];
    sig[c] = std::sqrt(std::max(lam[src], 0.0));
  }
  if (sig[0] > 0) {
    for (int c = 0; c < bs; ++c) sig[c] = std::max(sig[c], 1e-12 * sig[0]);
  } else {
    for (int c = 0; c < bs; ++c) sig[c] = 1.0;
  }
  // Linv = L^{-1} (lower triangular), column by column forward substitution
  for (int j = 0; j < bs; ++j) {
    for (int i = 0; i < bs; ++i) {
      double s = (i == j) ? 1.0 : 0.0;
      for (int k = 0; k < i; ++k) s -= L[i * bs + k] * Linv[k * bs + j];
      Linv[i * bs + j] = (i < j) ? 0.0 : s / L[i * bs + i];
    }
  }
  // Mx = S^{-1/2} U^T L^T,  Mw = S^{1/2} U^T L^{-1}
  std::vector<double> Mx(bs * bs), Mw(bs * bs);
  for (int i = 0; i < bs; ++i) {
    double rx = 1.0 / std::sqrt(sig[i]), rw = std::sqrt(sig[i]);
    for (int j = 0; j < bs; ++j) {
      double sx = 0.0, sw = 0.0;
      for (int k = 0; k < bs; ++k) {
        sx += U[k * bs + i] * L[j * bs + k];
        sw += U[k * bs + i] * Linv[k * bs + j];
      }
      Mx[i * bs + j] = rx * sx;
      Mw[i * bs + j] = rw * sw;
    }
  }
  if (!with_h) {
    std::memcpy(tx, Mx.data(), sizeof(double) * bs * bs);
    std::memcpy(tw, Mw.data(), sizeof(double) * bs * bs);
    return true;
  }
  for (int i = 0; i < bs; ++i)
    for (int j = 0; j < bs; ++j) {
      double sx = 0.0, sw = 0.0;
      for (int k = 0; k < bs; ++k) {
        double h = hadamard_entry(i, k, bs);
        sx += h * Mx[k * bs + j];
        sw += h * Mw[k * bs + j];
      }
      tx[i * bs + j] = sx;
      tw[i * bs + j] = sw;
    }
  return true;
}

}  // namespace
}  // namespace wush

using wush::fail;

namespace {
constexpr double kHdFloor = 1e-12;   // moments below this fraction of the block's largest are floored
}

extern "C" {

const char* wush_status_string(wush_status s) {
  switch (s) {
    case WUSH_OK: return "ok";
    case WUSH_E_ARG: return "invalid argument";
    case WUSH_E_SHAPE: return "invalid shape";
    case WUSH_E_NUMERIC: return "numerical failure";
    case WUSH_E_HIP: return "HIP runtime error";
    case WUSH_E_UNSUPPORTED: return "unsupported";
  }
  return "unknown status";
}

const char* wush_last_error(void) { return wush::g_last_error.c_str(); }

const char* wush_version(void) { return "wush 0.1 gfx950"; }

int wush_format_block(wush_format fmt) {
  switch (fmt) {
    case WUSH_MXFP4: return 32;
    case WUSH_NVFP4: return 16;
    case WUSH_INT4: return 32;
  }
  return 0;
}

wush_status wush_block_moments(int bs, int n, int d_in, const float* X, float* Sx) {
  WUSH_REQUIRE(X && Sx, WUSH_E_ARG, "wush_block_moments: null pointer");
  WUSH_REQUIRE(bs == 16 || bs == 32, WUSH_E_SHAPE, "wush_block_moments: bs must be 16 or 32 (got %d)", bs);
  WUSH_REQUIRE(n >= 1 && d_in >= bs && d_in % bs == 0, WUSH_E_SHAPE,
               "wush_block_moments: need n >= 1 and d_in %% bs == 0 (n=%d d_in=%d bs=%d)", n, d_in, bs);
  const int nblk = d_in / bs;
  wush::parallel_blocks(nblk, [&](int b) {
    std::vector<double> acc(bs * bs, 0.0);
    for (int t = 0; t < n; ++t) {
      const float* x = X + static_cast<size_t>(t) * d_in + static_cast<size_t>(b) * bs;
      for (int i = 0; i < bs; ++i) {
        double xi = x[i];
        for (int j = 0; j <= i; ++j) acc[i * bs + j] += xi * static_cast<double>(x[j]);
      }
    }
    float* out = Sx + static_cast<size_t>(b) * bs * bs;
    for (int i = 0; i < bs; ++i)
      for (int j = 0; j <= i; ++j) {
        float v = static_cast<float>(acc[i * bs + j] / n);
        out[i * bs + j] = v;
        out[j * bs + i] = v;
      }
  });
  return WUSH_OK;
}

wush_status wush_build_transforms(wush_kind kind, int bs, int d_in, int d_out, const float* W,
                                  const float* Sx, float* Tx, float* Tw) {
  WUSH_REQUIRE(Tx && Tw, WUSH_E_ARG, "wush_build_transforms: null output pointer");
  WUSH_REQUIRE(kind >= WUSH_IDENTITY && kind <= WUSH_WUSH, WUSH_E_ARG, "wush_build_transforms: bad kind %d",
               static_cast<int>(kind));
  WUSH_REQUIRE(bs == 16 || bs == 32, WUSH_E_SHAPE, "wush_build_transforms: bs must be 16 or 32 (got %d)", bs);
  WUSH_REQUIRE(d_in >= bs && d_in % bs == 0, WUSH_E_SHAPE, "wush_build_transforms: d_in %% bs != 0 (d_in=%d)",
               d_in);
  const int nblk = d_in / bs;
  const size_t msz = static_cast<size_t>(bs) * bs;
  if (kind == WUSH_IDENTITY || kind == WUSH_HADAMARD) {
    for (int b = 0; b < nblk; ++b)
      for (int i = 0; i < bs; ++i)
        for (int j = 0; j < bs; ++j) {
          float v = kind == WUSH_IDENTITY ? (i == j ? 1.0f : 0.0f)
                                          : static_cast<float>(wush::hadamard_entry(i, j, bs));
          Tx[b * msz + i * bs + j] = v;
          Tw[b * msz + i * bs + j] = v;
        }
    return WUSH_OK;
  }
  WUSH_REQUIRE(W && Sx, WUSH_E_ARG, "wush_build_transforms: W and Sx are required for WUS/WUSH");
  WUSH_REQUIRE(d_out >= 1, WUSH_E_SHAPE, "wush_build_transforms: d_out must be >= 1");
  std::atomic<int> bad_block{-1};
  wush::parallel_blocks(nblk, [&](int b) {
    std::vector<double> A(msz, 0.0), B(msz), tx(msz), tw(msz);
    for (int o = 0; o < d_out; ++o) {
      const float* w = W + static_cast<size_t>(o) * d_in + static_cast<size_t>(b) * bs;
      for (int i = 0; i < bs; ++i) {
        double wi = w[i];
        for (int j = 0; j <= i; ++j) A[i * bs + j] += wi * static_cast<double>(w[j]);
      }
    }
    for (int i = 0; i < bs; ++i)
      for (int j = 0; j < i; ++j) A[j * bs + i] = A[i * bs + j];
    for (size_t i = 0; i < msz; ++i) B[i] = Sx[b * msz + i];
    if (!wush::block_transform(kind == WUSH_WUSH, bs, A.data(), B.data(), tx.data(), tw.data())) {
      bad_block = b;
      return;
    }
    for (size_t i = 0; i < msz; ++i) {
      Tx[b * msz + i] = static_cast<float>(tx[i]);
      Tw[b * msz + i] = static_cast<float>(tw[i]);
    }
  });
  if (bad_block.load() >= 0)
    return fail(WUSH_E_NUMERIC, "wush_build_transforms: block %d weight moment not positive definite after damping",
                bad_block.load());
  return WUSH_OK;
}

// Hadamard-diagonal variant (news article, deployment and limitation
// paragraphs: the data-aware component approximated by a diagonal matrix).
// From the moment diagonals a_i = sum_o W[o][i]^2 and b_i = Sx_b[i][i]:
// d_x = sqrt(sqrt(a / b)) / sqrt(bs), d_w = sqrt(sqrt(b / a)) / sqrt(bs),
// the optimum of the proxy among Hadamard-times-diagonal transforms.
wush_status wush_build_shared(wush_kind kind, int bs, int d_in, int d_out, const float* W, const float* Sx,
                              int ngroups, const int* group, float* Tx, float* Tw) {
  WUSH_REQUIRE(Tx && Tw && group, WUSH_E_ARG, "wush_build_shared: null pointer");
  WUSH_REQUIRE(kind >= WUSH_IDENTITY && kind <= WUSH_WUSH, WUSH_E_ARG, "wush_build_shared: bad kind %d",
               static_cast<int>(kind));
  WUSH_REQUIRE(bs == 16 || bs == 32, WUSH_E_SHAPE, "wush_build_shared: bs must be 16 or 32 (got %d)", bs);
  WUSH_REQUIRE(d_in >= bs && d_in % bs == 0, WUSH_E_SHAPE, "wush_build_shared: d_in %% bs != 0 (d_in=%d)", d_in);
  const int nblk = d_in / bs;
  WUSH_REQUIRE(ngroups >= 1 && ngroups <= nblk, WUSH_E_ARG, "wush_build_shared: need 1 <= ngroups <= %d", nblk);
  std::vector<int> count(ngroups, 0);
  for (int b = 0; b < nblk; ++b) {
    WUSH_REQUIRE(group[b] >= 0 && group[b] < ngroups, WUSH_E_ARG, "wush_build_shared: block %d has group %d", b,
                 group[b]);
    ++count[group[b]];
  }
  for (int gi = 0; gi < ngroups; ++gi)
    WUSH_REQUIRE(count[gi] > 0, WUSH_E_ARG, "wush_build_shared: group %d owns no block", gi);
  const size_t msz = static_cast<size_t>(bs) * bs;
  if (kind == WUSH_IDENTITY || kind == WUSH_HADAMARD)   // data-free: every group gets the same matrix
    return wush_build_transforms(kind, bs, ngroups * bs, d_out, nullptr, nullptr, Tx, Tw);
  WUSH_REQUIRE(W && Sx, WUSH_E_ARG, "wush_build_shared: W and Sx are required for WUS/WUSH");
  WUSH_REQUIRE(d_out >= 1, WUSH_E_SHAPE, "wush_build_shared: d_out must be >= 1");
  // per-block weight moments (fp64), then the sums over each group's blocks in block order
  std::vector<double> Ab(static_cast<size_t>(nblk) * msz, 0.0);
  wush::parallel_blocks(nblk, [&](int b) {
    double* A = Ab.data() + static_cast<size_t>(b) * msz;
    for (int o = 0; o < d_out; ++o) {
      const float* w = W + static_cast<size_t>(o) * d_in + static_cast<size_t>(b) * bs;
      for (int i = 0; i < bs; ++i) {
        const double wi = w[i];
        for (int j = 0; j <= i; ++j) A[i * bs + j] += wi * static_cast<double>(w[j]);
      }
    }
    for (int i = 0; i < bs; ++i)
      for (int j = 0; j < i; ++j) A[j * bs + i] = A[i * bs + j];
  });
  std::atomic<int> bad_group{-1};
  wush::parallel_blocks(ngroups, [&](int gi) {
    std::vector<double> A(msz, 0.0), B(msz, 0.0), tx(msz), tw(msz);
    for (int b = 0; b < nblk; ++b) {
      if (group[b] != gi) continue;
      const double* a = Ab.data() + static_cast<size_t>(b) * msz;
      for (size_t i = 0; i < msz; ++i) {
        A[i] += a[i];
        B[i] += Sx[static_cast<size_t>(b) * msz + i];
      }
    }
    if (!wush::block_transform(kind == WUSH_WUSH, bs, A.data(), B.data(), tx.data(), tw.data())) {
      bad_group = gi;
      return;
    }
    for (size_t i = 0; i < msz; ++i) {
      Tx[gi * msz + i] = static_cast<float>(tx[i]);
      Tw[gi * msz + i] = static_cast<float>(tw[i]);
    }
  });
  if (bad_group.load() >= 0)
    return fail(WUSH_E_NUMERIC, "wush_build_shared: group %d weight moment not positive definite after damping",
                bad_group.load());
  return WUSH_OK;
}

wush_status wush_build_hd(int bs, int d_in, int d_out, const float* W, const float* Sx, float* dx, float* dw) {
  WUSH_REQUIRE(W && Sx && dx && dw, WUSH_E_ARG, "wush_build_hd: null pointer");
  WUSH_REQUIRE(bs == 16 || bs == 32, WUSH_E_SHAPE, "wush_build_hd: bs must be 16 or 32 (got %d)", bs);
  WUSH_REQUIRE(d_in >= bs && d_in % bs == 0, WUSH_E_SHAPE, "wush_build_hd: d_in %% bs != 0 (d_in=%d)", d_in);
  WUSH_REQUIRE(d_out >= 1, WUSH_E_SHAPE, "wush_build_hd: d_out must be >= 1");
  const int nblk = d_in / bs;
  const double inv = 1.0 / std::sqrt(static_cast<double>(bs));
  std::atomic<int> bad_block{-1};
  wush::parallel_blocks(nblk, [&](int b) {
    std::vector<double> a(bs, 0.0), s(bs);
    for (int o = 0; o < d_out; ++o) {
      const float* w = W + static_cast<size_t>(o) * d_in + static_cast<size_t>(b) * bs;
      for (int i = 0; i < bs; ++i) a[i] += static_cast<double>(w[i]) * static_cast<double>(w[i]);
    }
    double amax = 0.0, smax = 0.0;
    for (int i = 0; i < bs; ++i) {
      s[i] = Sx[(static_cast<size_t>(b) * bs + i) * bs + i];
      amax = std::max(amax, a[i]);
      smax = std::max(smax, s[i]);
    }
    if (!(amax > 0.0)) {
      bad_block = b;
      return;
    }
    for (int i = 0; i < bs; ++i) {
      const double ai = std::max(a[i], kHdFloor * amax);
      const double si = smax > 0.0 ? std::max(s[i], kHdFloor * smax) : 1.0;
      dx[b * bs + i] = static_cast<float>(std::sqrt(std::sqrt(ai / si)) * inv);
      dw[b * bs + i] = static_cast<float>(std::sqrt(std::sqrt(si / ai)) * inv);
    }
  });
  if (bad_block.load() >= 0)
    return fail(WUSH_E_NUMERIC, "wush_build_hd: block %d has all-zero weights", bad_block.load());
  return WUSH_OK;
}

}  // extern "C"
