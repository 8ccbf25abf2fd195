// The transform builder on the GPU: per-block weight moments, damped
// Cholesky, C = W'^T B W', cyclic Jacobi eigen-decomposition and the two
// transforms, for all blocks at once.
//
// WUSH news article, construction paragraph (Cholesky factor of the weight
// statistics, SVD, Hadamard) and deployment paragraph (the per-block
// computations are independent and run in parallel).
//
// Same algorithm, operation order and fp64 arithmetic as the host builder
// (builder.cpp, compiled without contraction like this file): the weight
// moment sums run over the rows in order, one thread per matrix entry, and
// each block's factorisations run in one thread, so both builders produce the
// same matrices.  It is an offline step (the pages put it before inference);
// the point of running it here is to keep W and the moments on the device.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.h"

namespace {

constexpr int kMaxBs = 32;
constexpr int kMaxSq = kMaxBs * kMaxBs;

// A[b][i][j] (j <= i, then mirrored) = sum over rows o in order of w_i w_j (fp64)
__global__ void weight_moments_kernel(const float* __restrict__ W, int d_out, int d_in, int bs,
                                      double* __restrict__ A) {
  const int nblk = d_in / bs;
  const int pairs = bs * (bs + 1) / 2;
  const long id = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (id >= static_cast<long>(nblk) * pairs) return;
  const int b = static_cast<int>(id / pairs);
  int p = static_cast<int>(id % pairs), i = 0;
  while (p > i) { p -= i + 1; ++i; }          // (i, j) with j = p <= i
  const int j = p;
  const float* w = W + static_cast<size_t>(b) * bs;
  double s = 0.0;
  for (int o = 0; o < d_out; ++o) {
    const double wi = w[static_cast<size_t>(o) * d_in + i];
    s += wi * static_cast<double>(w[static_cast<size_t>(o) * d_in + j]);
  }
  double* Ab = A + static_cast<size_t>(b) * bs * bs;
  Ab[i * bs + j] = s;
  Ab[j * bs + i] = s;
}

__device__ bool cholesky_lower(double* a, int bs) {
  for (int j = 0; j < bs; ++j) {
    double d = a[j * bs + j];
    for (int k = 0; k < j; ++k) d -= a[j * bs + k] * a[j * bs + k];
    if (!(d > 0.0)) return false;
    const double ljj = sqrt(d);
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

// cyclic Jacobi; a is destroyed, lam the eigenvalues, column i of v its vector
__device__ void jacobi_eigh(double* a, int bs, double* lam, double* v) {
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
        const double apq = a[p * bs + q];
        if (apq == 0.0) continue;
        const double app = a[p * bs + p], aqq = a[q * bs + q];
        const double theta = (aqq - app) / (2.0 * apq);
        const double t = (theta >= 0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
        const double c = 1.0 / sqrt(t * t + 1.0);
        const double s = t * c;
        for (int k = 0; k < bs; ++k) {
          const double akp = a[k * bs + p], akq = a[k * bs + q];
          a[k * bs + p] = c * akp - s * akq;
          a[k * bs + q] = s * akp + c * akq;
        }
        for (int k = 0; k < bs; ++k) {
          const double apk = a[p * bs + k], aqk = a[q * bs + k];
          a[p * bs + k] = c * apk - s * aqk;
          a[q * bs + k] = s * apk + c * aqk;
        }
        a[p * bs + q] = a[q * bs + p] = 0.0;
        for (int k = 0; k < bs; ++k) {
          const double vkp = v[k * bs + p], vkq = v[k * bs + q];
          v[k * bs + p] = c * vkp - s * vkq;
          v[k * bs + q] = s * vkp + c * vkq;
        }
      }
    }
  }
  for (int i = 0; i < bs; ++i) lam[i] = a[i * bs + i];
}

__device__ double hadamard_entry(int i, int j, int bs) {
  return (__builtin_popcount(static_cast<unsigned>(i & j)) & 1 ? -1.0 : 1.0) / sqrt(static_cast<double>(bs));
}

// One block per workgroup, worked by its first lane with its matrices in the
// workgroup's LDS (41 KB; as private arrays they would need 41 KB of scratch
// per lane): kind 0 identity, 1 Hadamard, 2 WUS, 3 WUSH (wush_kind).
// status[b] = 1 when no rung of the damping ladder gives a Cholesky factor.
__global__ __launch_bounds__(64) void build_blocks_kernel(int kind, int bs, int nblk, const double* __restrict__ Aall,
                                                          const float* __restrict__ Sx, float* __restrict__ Tx,
                                                          float* __restrict__ Tw, int* __restrict__ status) {
  __shared__ double L[kMaxSq], C[kMaxSq], M1[kMaxSq], V[kMaxSq], M2[kMaxSq], lam[kMaxBs], sig[kMaxBs];
  __shared__ int order[kMaxBs];
  const int b = blockIdx.x;
  if (b >= nblk || threadIdx.x != 0) return;   // no barrier below
  const int sq = bs * bs;
  float* tx = Tx + static_cast<size_t>(b) * sq;
  float* tw = Tw + static_cast<size_t>(b) * sq;
  status[b] = 0;
  if (kind == WUSH_IDENTITY || kind == WUSH_HADAMARD) {
    for (int i = 0; i < bs; ++i)
      for (int j = 0; j < bs; ++j) {
        const float v = kind == WUSH_IDENTITY ? (i == j ? 1.0f : 0.0f) : static_cast<float>(hadamard_entry(i, j, bs));
        tx[i * bs + j] = v;
        tw[i * bs + j] = v;
      }
    return;
  }
  const double* A = Aall + static_cast<size_t>(b) * sq;
  const float* B = Sx + static_cast<size_t>(b) * sq;
  double tr = 0.0;
  for (int i = 0; i < bs; ++i) tr += A[i * bs + i];
  const double damping[] = {0.0, 1e-10, 1e-8, 1e-6, 1e-4, 1e-2};
  bool ok = false;
  for (int r = 0; r < 6 && !ok; ++r) {
    for (int i = 0; i < sq; ++i) L[i] = A[i];
    for (int i = 0; i < bs; ++i) L[i * bs + i] += damping[r] * (tr / bs);
    ok = cholesky_lower(L, bs);
  }
  if (!ok) {
    status[b] = 1;
    return;
  }
  // C = L^T B L (symmetrised); M1 holds B L
  for (int i = 0; i < bs; ++i)
    for (int j = 0; j < bs; ++j) {
      double s = 0.0;
      for (int k = 0; k < bs; ++k) s += static_cast<double>(B[i * bs + k]) * L[k * bs + j];
      M1[i * bs + j] = s;
    }
  for (int i = 0; i < bs; ++i)
    for (int j = 0; j < bs; ++j) {
      double s = 0.0;
      for (int k = 0; k < bs; ++k) s += L[k * bs + i] * M1[k * bs + j];
      C[i * bs + j] = s;
    }
  for (int i = 0; i < bs; ++i)
    for (int j = i + 1; j < bs; ++j) {
      const double m = 0.5 * (C[i * bs + j] + C[j * bs + i]);
      C[i * bs + j] = C[j * bs + i] = m;
    }
  jacobi_eigh(C, bs, lam, V);
  // eigenvalues descending, ties in index order (a stable insertion sort)
  for (int i = 0; i < bs; ++i) {
    int k = i;
    while (k > 0 && lam[i] > lam[order[k - 1]]) {
      order[k] = order[k - 1];
      --k;
    }
    order[k] = i;
  }
  // U (in C): columns sorted, each signed so its largest-magnitude entry is positive
  for (int c = 0; c < bs; ++c) {
    const int src = order[c];
    int piv = 0;
    for (int r = 1; r < bs; ++r)
      if (fabs(V[r * bs + src]) > fabs(V[piv * bs + src])) piv = r;
    const double sg = V[piv * bs + src] < 0 ? -1.0 : 1.0;
    for (int r = 0; r < bs; ++r) C[r * bs + c] = sg * V[r * bs + src];
    sig[c] = sqrt(fmax(lam[src], 0.0));
  }
  if (sig[0] > 0) {
    for (int c = 0; c < bs; ++c) sig[c] = fmax(sig[c], 1e-12 * sig[0]);
  } else {
    for (int c = 0; c < bs; ++c) sig[c] = 1.0;
  }
  // M1 = L^{-1} (lower triangular), column by column forward substitution
  for (int j = 0; j < bs; ++j)
    for (int i = 0; i < bs; ++i) {
      double s = (i == j) ? 1.0 : 0.0;
      for (int k = 0; k < i; ++k) s -= L[i * bs + k] * M1[k * bs + j];
      M1[i * bs + j] = (i < j) ? 0.0 : s / L[i * bs + i];
    }
  // V = Mx = S^{-1/2} U^T L^T,  M2 = Mw = S^{1/2} U^T L^{-1}
  for (int i = 0; i < bs; ++i) {
    const double rx = 1.0 / sqrt(sig[i]), rw = sqrt(sig[i]);
    for (int j = 0; j < bs; ++j) {
      double sx = 0.0, sw = 0.0;
      for (int k = 0; k < bs; ++k) {
        sx += C[k * bs + i] * L[j * bs + k];
        sw += C[k * bs + i] * M1[k * bs + j];
      }
      V[i * bs + j] = rx * sx;
      M2[i * bs + j] = rw * sw;
    }
  }
  if (kind != WUSH_WUSH) {   // WUS: no Hadamard
    for (int i = 0; i < sq; ++i) {
      tx[i] = static_cast<float>(V[i]);
      tw[i] = static_cast<float>(M2[i]);
    }
    return;
  }
  for (int i = 0; i < bs; ++i)
    for (int j = 0; j < bs; ++j) {
      double sx = 0.0, sw = 0.0;
      for (int k = 0; k < bs; ++k) {
        const double h = hadamard_entry(i, k, bs);
        sx += h * V[k * bs + j];
        sw += h * M2[k * bs + j];
      }
      tx[i * bs + j] = static_cast<float>(sx);
      tw[i * bs + j] = static_cast<float>(sw);
    }
}

}  // namespace

extern "C" {

size_t wush_build_transforms_dev_ws_bytes(int bs, int d_in) {
  if ((bs != 16 && bs != 32) || d_in < bs || d_in % bs != 0) return 0;
  const size_t nblk = d_in / bs;
  return nblk * bs * bs * sizeof(double) + ((nblk * sizeof(int) + 255) / 256) * 256;
}

wush_status wush_build_transforms_dev(wush_kind kind, int bs, int d_in, int d_out, const float* W, const float* Sx,
                                      float* Tx, float* Tw, void* ws, size_t ws_bytes, void* stream) {
  if (kind < WUSH_IDENTITY || kind > WUSH_WUSH)
    return wush::fail(WUSH_E_ARG, "wush_build_transforms_dev: bad kind %d", static_cast<int>(kind));
  if ((bs != 16 && bs != 32) || d_in < bs || d_in % bs != 0)
    return wush::fail(WUSH_E_SHAPE, "wush_build_transforms_dev: bs 16 or 32 and d_in a multiple of bs");
  if (!Tx || !Tw) return wush::fail(WUSH_E_ARG, "wush_build_transforms_dev: null output pointer");
  const bool data = kind == WUSH_WUS || kind == WUSH_WUSH;
  if (data && (!W || !Sx)) return wush::fail(WUSH_E_ARG, "wush_build_transforms_dev: W and Sx are required");
  if (data && d_out < 1) return wush::fail(WUSH_E_SHAPE, "wush_build_transforms_dev: d_out must be >= 1");
  const size_t need = wush_build_transforms_dev_ws_bytes(bs, d_in);
  if (!ws || ws_bytes < need || !wush::aligned16(ws))
    return wush::fail(WUSH_E_ARG, "wush_build_transforms_dev: workspace of %zu bytes (16-byte aligned) needed", need);
  const int nblk = d_in / bs;
  hipStream_t s = static_cast<hipStream_t>(stream);
  double* A = static_cast<double*>(ws);
  int* status = reinterpret_cast<int*>(static_cast<uint8_t*>(ws) + static_cast<size_t>(nblk) * bs * bs * sizeof(double));
  if (data) {
    const long threads = static_cast<long>(nblk) * (bs * (bs + 1) / 2);
    hipLaunchKernelGGL(weight_moments_kernel, dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, s, W,
                       d_out, d_in, bs, A);
  }
  hipLaunchKernelGGL(build_blocks_kernel, dim3(nblk), dim3(64), 0, s, static_cast<int>(kind), bs, nblk, A,
                     Sx, Tx, Tw, status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return wush::fail(WUSH_E_HIP, "wush_build_transforms_dev launch: %s", hipGetErrorString(e));
  // the damping results come back to the host (this call synchronises the stream)
  int* hs = new int[nblk];
  e = hipMemcpyAsync(hs, status, sizeof(int) * nblk, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  int bad = -1;
  for (int b = 0; b < nblk && e == hipSuccess; ++b)
    if (hs[b]) { bad = b; break; }
  delete[] hs;
  if (e != hipSuccess) return wush::fail(WUSH_E_HIP, "wush_build_transforms_dev: %s", hipGetErrorString(e));
  if (bad >= 0)
    return wush::fail(WUSH_E_NUMERIC, "wush_build_transforms_dev: block %d weight moment not positive definite after "
                      "damping", bad);
  return WUSH_OK;
}

}  // extern "C"
