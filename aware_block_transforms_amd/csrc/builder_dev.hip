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
// each block's factorisations run in one wave whose lanes split the entries
// that do not depend on each other, every entry computed from the same
// operands in the same order as on the host, so both builders produce the
// same matrices.  It is an offline step (the pages put it before inference);
// the point of running it here is to keep W and the moments on the device.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.h"

namespace {

constexpr int kMaxBs = 32;
constexpr int kMaxSq = kMaxBs * kMaxBs;

// A[b][i][j] (j <= i, then mirrored) = sum over rows o in order of w_i w_j
// (fp64).  One workgroup per block: the block's bs columns of W pass through
// LDS kMomRows rows at a time (two buffers; the next chunk is loaded into
// registers before the current one is summed and stored after it), and
// thread t keeps the sums of lower-triangle entries 2t and 2t + 1, each over
// the rows in order.
constexpr int kMomRows = 64;
constexpr int kMomPer = 8;    // chunk elements per thread: kMomRows * bs / threads, at most 8

__device__ __forceinline__ void moment_entry(int p, int& i, int& j) {
  i = 0;
  while (p > i) { p -= i + 1; ++i; }          // (i, j) with j = p <= i
  j = p;
}

__global__ __launch_bounds__(320) void weight_moments_kernel(const float* __restrict__ W, int d_out, int d_in, int bs,
                                                             double* __restrict__ A) {
  __shared__ float rows[2][kMomRows * kMaxBs];
  const int b = blockIdx.x, t = threadIdx.x, nt = blockDim.x;
  const int pairs = bs * (bs + 1) / 2;
  const bool has0 = 2 * t < pairs, has1 = 2 * t + 1 < pairs;
  int i0 = 0, j0 = 0, i1 = 0, j1 = 0;
  if (has0) moment_entry(2 * t, i0, j0);
  if (has1) moment_entry(2 * t + 1, i1, j1);
  const float* Wb = W + static_cast<size_t>(b) * bs;
  const int pieces = kMomRows * bs;
  float pre[kMomPer];
  auto fetch = [&](int o0) {
#pragma unroll
    for (int k = 0; k < kMomPer; ++k) {
      const int pc = t + k * nt, r = pc / bs, c = pc % bs;
      pre[k] = pc < pieces && o0 + r < d_out ? Wb[static_cast<size_t>(o0 + r) * d_in + c] : 0.0f;
    }
  };
  auto put = [&](int buf) {
#pragma unroll
    for (int k = 0; k < kMomPer; ++k)
      if (t + k * nt < pieces) rows[buf][t + k * nt] = pre[k];
  };
  double s0 = 0.0, s1 = 0.0;
  fetch(0);
  put(0);
  __syncthreads();
  int buf = 0;
  for (int o0 = 0; o0 < d_out; o0 += kMomRows) {
    const bool more = o0 + kMomRows < d_out;
    if (more) fetch(o0 + kMomRows);
    const int nr = min(kMomRows, d_out - o0);
    const float* w = rows[buf];
    for (int r = 0; r < nr; ++r, w += bs) {
      const double wi0 = w[i0];
      s0 += wi0 * static_cast<double>(w[j0]);
      const double wi1 = w[i1];
      s1 += wi1 * static_cast<double>(w[j1]);
    }
    if (more) put(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
  double* Ab = A + static_cast<size_t>(b) * bs * bs;
  if (has0) { Ab[i0 * bs + j0] = s0; Ab[j0 * bs + i0] = s0; }
  if (has1) { Ab[i1 * bs + j1] = s1; Ab[j1 * bs + i1] = s1; }
}

// Workgroup barrier with LDS completion (the workgroup is one wave, so the
// barrier itself is immediate; the wait makes this lane's LDS writes visible).
__device__ __forceinline__ void sync_lds() { __syncthreads(); }

// Lower Cholesky factor in place (upper part zeroed), or false.  Column j:
// every lane forms the pivot d from row j in order (the same value in every
// lane), then lane i (i > j) forms row i's entry from its own row and row j,
// in order.
__device__ bool cholesky_lower(double* a, int bs, int t) {
  for (int j = 0; j < bs; ++j) {
    double d = a[j * bs + j];
    for (int k = 0; k < j; ++k) d -= a[j * bs + k] * a[j * bs + k];
    if (!(d > 0.0)) return false;   // the same in every lane
    const double ljj = sqrt(d);
    double s = 0.0;
    if (t > j && t < bs) {
      s = a[t * bs + j];
      for (int k = 0; k < j; ++k) s -= a[t * bs + k] * a[j * bs + k];
    }
    sync_lds();
    if (t == j) a[j * bs + j] = ljj;
    if (t > j && t < bs) {
      a[t * bs + j] = s / ljj;
      a[j * bs + t] = 0.0;
    }
    sync_lds();
  }
  return true;
}

// Cyclic Jacobi; a is destroyed, lam the eigenvalues, column i of v its
// vector.  The rotations run in the host's (p, q) order; every lane computes
// each rotation's c and s from the same three entries, then lane k applies it
// to column entries (k, p), (k, q) of a and v, and after a barrier to row
// entries (p, k), (q, k).  The two entries the host zeroes after the rotation
// are stored as zero directly (the values they would have taken are never
// read).
__device__ void jacobi_eigh(double* a, int bs, double* lam, double* v, int t) {
  for (int e = t; e < bs * bs; e += 64) v[e] = (e / bs == e % bs) ? 1.0 : 0.0;
  sync_lds();
  for (int sweep = 0; sweep < 100; ++sweep) {
    double off = 0.0, diag = 0.0;
    for (int p = 0; p < bs; ++p) {
      diag += a[p * bs + p] * a[p * bs + p];
      for (int q = p + 1; q < bs; ++q) off += a[p * bs + q] * a[p * bs + q];
    }
    if (off <= 1e-34 * diag || off == 0.0) break;   // the same in every lane
    for (int p = 0; p < bs - 1; ++p) {
      for (int q = p + 1; q < bs; ++q) {
        const double apq = a[p * bs + q];
        if (apq == 0.0) continue;
        const double app = a[p * bs + p], aqq = a[q * bs + q];
        const double theta = (aqq - app) / (2.0 * apq);
        const double tt = (theta >= 0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
        const double c = 1.0 / sqrt(tt * tt + 1.0);
        const double s = tt * c;
        sync_lds();
        if (t < bs) {
          const double akp = a[t * bs + p], akq = a[t * bs + q];
          a[t * bs + p] = c * akp - s * akq;
          a[t * bs + q] = s * akp + c * akq;
          const double vkp = v[t * bs + p], vkq = v[t * bs + q];
          v[t * bs + p] = c * vkp - s * vkq;
          v[t * bs + q] = s * vkp + c * vkq;
        }
        sync_lds();
        if (t < bs) {
          const double apk = a[p * bs + t], aqk = a[q * bs + t];
          a[p * bs + t] = t == q ? 0.0 : c * apk - s * aqk;
          a[q * bs + t] = t == p ? 0.0 : s * apk + c * aqk;
        }
        sync_lds();
      }
    }
  }
  if (t < bs) lam[t] = a[t * bs + t];
  sync_lds();
}

__device__ double hadamard_entry(int i, int j, int bs) {
  return (__builtin_popcount(static_cast<unsigned>(i & j)) & 1 ? -1.0 : 1.0) / sqrt(static_cast<double>(bs));
}

// One block per workgroup of one wave, its matrices in the workgroup's LDS
// (41 KB): kind 0 identity, 1 Hadamard, 2 WUS, 3 WUSH (wush_kind).
// status[b] = 1 when no rung of the damping ladder gives a Cholesky factor.
// Every branch below is uniform across the wave, so every lane reaches every
// barrier.
__global__ __launch_bounds__(64) void build_blocks_kernel(int kind, int bs, int nblk, const double* __restrict__ Aall,
                                                          const float* __restrict__ Sx, float* __restrict__ Tx,
                                                          float* __restrict__ Tw, int* __restrict__ status) {
  __shared__ double L[kMaxSq], C[kMaxSq], M1[kMaxSq], V[kMaxSq], M2[kMaxSq], lam[kMaxBs], sig[kMaxBs];
  __shared__ int order[kMaxBs];
  const int b = blockIdx.x;
  if (b >= nblk) return;   // workgroup-uniform
  const int t = threadIdx.x;
  const int sq = bs * bs;
  float* tx = Tx + static_cast<size_t>(b) * sq;
  float* tw = Tw + static_cast<size_t>(b) * sq;
  if (t == 0) status[b] = 0;
  if (kind == WUSH_IDENTITY || kind == WUSH_HADAMARD) {
    for (int e = t; e < sq; e += 64) {
      const int i = e / bs, j = e % bs;
      const float v = kind == WUSH_IDENTITY ? (i == j ? 1.0f : 0.0f) : static_cast<float>(hadamard_entry(i, j, bs));
      tx[e] = v;
      tw[e] = v;
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
    for (int e = t; e < sq; e += 64) L[e] = A[e];
    sync_lds();
    if (t < bs) L[t * bs + t] += damping[r] * (tr / bs);
    sync_lds();
    ok = cholesky_lower(L, bs, t);
  }
  if (!ok) {
    if (t == 0) status[b] = 1;
    return;
  }
  // C = L^T B L (symmetrised); M1 holds B L
  for (int e = t; e < sq; e += 64) {
    const int i = e / bs, j = e % bs;
    double s = 0.0;
    for (int k = 0; k < bs; ++k) s += static_cast<double>(B[i * bs + k]) * L[k * bs + j];
    M1[e] = s;
  }
  sync_lds();
  for (int e = t; e < sq; e += 64) {
    const int i = e / bs, j = e % bs;
    double s = 0.0;
    for (int k = 0; k < bs; ++k) s += L[k * bs + i] * M1[k * bs + j];
    C[e] = s;
  }
  sync_lds();
  for (int e = t; e < sq; e += 64) {
    const int i = e / bs, j = e % bs;
    if (j > i) {   // each pair (i, j), j > i, by one lane
      const double m = 0.5 * (C[i * bs + j] + C[j * bs + i]);
      C[i * bs + j] = C[j * bs + i] = m;
    }
  }
  sync_lds();
  jacobi_eigh(C, bs, lam, V, t);
  // eigenvalues descending, ties in index order (a stable insertion sort)
  if (t == 0) {
    for (int i = 0; i < bs; ++i) {
      int k = i;
      while (k > 0 && lam[i] > lam[order[k - 1]]) {
        order[k] = order[k - 1];
        --k;
      }
      order[k] = i;
    }
  }
  sync_lds();
  // U (in C): columns sorted, each signed so its largest-magnitude entry is
  // positive; lane c takes column c
  if (t < bs) {
    const int src = order[t];
    int piv = 0;
    for (int r = 1; r < bs; ++r)
      if (fabs(V[r * bs + src]) > fabs(V[piv * bs + src])) piv = r;
    const double sg = V[piv * bs + src] < 0 ? -1.0 : 1.0;
    for (int r = 0; r < bs; ++r) C[r * bs + t] = sg * V[r * bs + src];
    sig[t] = sqrt(fmax(lam[src], 0.0));
  }
  sync_lds();
  const double sig0 = sig[0];
  sync_lds();
  if (t < bs) sig[t] = sig0 > 0 ? fmax(sig[t], 1e-12 * sig0) : 1.0;
  // M1 = L^{-1} (lower triangular), forward substitution; lane j takes column j
  if (t < bs) {
    const int j = t;
    for (int i = 0; i < bs; ++i) {
      double s = (i == j) ? 1.0 : 0.0;
      for (int k = 0; k < i; ++k) s -= L[i * bs + k] * M1[k * bs + j];
      M1[i * bs + j] = (i < j) ? 0.0 : s / L[i * bs + i];
    }
  }
  sync_lds();
  // V = Mx = S^{-1/2} U^T L^T,  M2 = Mw = S^{1/2} U^T L^{-1}
  for (int e = t; e < sq; e += 64) {
    const int i = e / bs, j = e % bs;
    const double rx = 1.0 / sqrt(sig[i]), rw = sqrt(sig[i]);
    double sx = 0.0, sw = 0.0;
    for (int k = 0; k < bs; ++k) {
      sx += C[k * bs + i] * L[j * bs + k];
      sw += C[k * bs + i] * M1[k * bs + j];
    }
    V[e] = rx * sx;
    M2[e] = rw * sw;
  }
  sync_lds();
  if (kind != WUSH_WUSH) {   // WUS: no Hadamard
    for (int e = t; e < sq; e += 64) {
      tx[e] = static_cast<float>(V[e]);
      tw[e] = static_cast<float>(M2[e]);
    }
    return;
  }
  for (int e = t; e < sq; e += 64) {
    const int i = e / bs, j = e % bs;
    double sx = 0.0, sw = 0.0;
    for (int k = 0; k < bs; ++k) {
      const double h = hadamard_entry(i, k, bs);
      sx += h * V[k * bs + j];
      sw += h * M2[k * bs + j];
    }
    tx[e] = static_cast<float>(sx);
    tw[e] = static_cast<float>(sw);
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
    const int threads = ((bs * (bs + 1) / 2 + 1) / 2 + 63) / 64 * 64;   // two entries per thread: 320 (bs 32), 128
    hipLaunchKernelGGL(weight_moments_kernel, dim3(nblk), dim3(threads), 0, s, W, d_out, d_in, bs, A);
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
