// Fixed (not generated) kernels of libcgtp for gfx950: real spherical
// harmonics of the edge vectors and the sender-sorted transpose of a
// receiver CSR.
//
// Spherical harmonics: the edge features of the convolution (sciencestack.ai
// page, Figure 4B).  Component normalisation, real basis with l = 1 ordered
// (y, z, x).  Evaluated with the reduced associated Legendre recurrence
// (no Condon-Shortley factor, which the real combination cancels) times the
// Chebyshev-like recurrence of r_xy^m cos(m phi) and r_xy^m sin(m phi).
//
// Receiver order: a stable bucket sort of the receivers by floor(log2(degree+1)),
// heaviest bucket first, so that long CSR rows start early (power-law graphs).
//
// Transpose: a stable counting sort of the edges by sender, needed by the
// atomic-free backward (OpenEquivariance discussion: a deterministic fused
// convolution next to the atomic one).  Counting uses integer atomics, whose
// totals are exact; the placement inside a sender is then sorted by edge id,
// so the result is unique and bit-exact.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <map>
#include <mutex>

#include "static_kernels.h"

namespace cgtp {

// ------------------------------------------------------------------------------------------
// spherical harmonics

template <typename T, int L>
__global__ void __launch_bounds__(256) sh_kernel(int64_t E, const T *__restrict__ vec, T *__restrict__ y)
{
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= E) return;
    constexpr int D = (L + 1) * (L + 1);
    T vx = vec[3 * e], vy = vec[3 * e + 1], vz = vec[3 * e + 2];
    T r2 = vx * vx + vy * vy + vz * vz;
    T inv = r2 > (T)0 ? (T)1 / sqrt(r2) : (T)0;
    T x = vx * inv, yy = vy * inv, z = vz * inv;
    T c[L + 1], s[L + 1];
    c[0] = (T)1;
    s[0] = (T)0;
#pragma unroll
    for (int m = 0; m < L; ++m) {
        c[m + 1] = x * c[m] - yy * s[m];
        s[m + 1] = x * s[m] + yy * c[m];
    }
    T out[D];
#pragma unroll
    for (int m = 0; m <= L; ++m) {
        // reduced Legendre Q_l^m(z), l = m..L
        T dfact = (T)1;
        for (int k = 1; k <= 2 * m - 1; k += 2) dfact *= (T)k;
        T qmm = dfact, q_prev = (T)0, q = qmm;
#pragma unroll
        for (int l = m; l <= L; ++l) {
            if (l == m) {
                q = qmm;
            } else if (l == m + 1) {
                q_prev = qmm;
                q = z * (T)(2 * m + 1) * qmm;
            } else {
                T qn = ((T)(2 * l - 1) * z * q - (T)(l + m - 1) * q_prev) / (T)(l - m);
                q_prev = q;
                q = qn;
            }
            // sqrt(2 (2l+1) (l-m)! / (l+m)!) for m > 0, sqrt(2l+1) for m = 0
            T ratio = (T)1;
            for (int k = l - m + 1; k <= l + m; ++k) ratio /= (T)k;
            if (m == 0) {
                out[l * l + l] = sqrt((T)(2 * l + 1)) * q;
            } else {
                T coef = sqrt((T)2 * (T)(2 * l + 1) * ratio) * q;
                out[l * l + l + m] = coef * c[m];
                out[l * l + l - m] = coef * s[m];
            }
        }
    }
#pragma unroll
    for (int i = 0; i < D; ++i) y[(size_t)e * D + i] = out[i];
}

template <typename T>
static hipError_t launch_sh_t(int lmax, int64_t E, const void *vec, void *y, hipStream_t st)
{
    dim3 grid((unsigned)((E + 255) / 256)), block(256);
    const T *v = static_cast<const T *>(vec);
    T *o = static_cast<T *>(y);
    switch (lmax) {
    case 0: hipLaunchKernelGGL((sh_kernel<T, 0>), grid, block, 0, st, E, v, o); break;
    case 1: hipLaunchKernelGGL((sh_kernel<T, 1>), grid, block, 0, st, E, v, o); break;
    case 2: hipLaunchKernelGGL((sh_kernel<T, 2>), grid, block, 0, st, E, v, o); break;
    case 3: hipLaunchKernelGGL((sh_kernel<T, 3>), grid, block, 0, st, E, v, o); break;
    case 4: hipLaunchKernelGGL((sh_kernel<T, 4>), grid, block, 0, st, E, v, o); break;
    case 5: hipLaunchKernelGGL((sh_kernel<T, 5>), grid, block, 0, st, E, v, o); break;
    case 6: hipLaunchKernelGGL((sh_kernel<T, 6>), grid, block, 0, st, E, v, o); break;
    case 7: hipLaunchKernelGGL((sh_kernel<T, 7>), grid, block, 0, st, E, v, o); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_spherical_harmonics(int lmax, bool f64, int64_t E, const void *vec, void *y, hipStream_t st)
{
    if (E == 0) return hipSuccess;
    return f64 ? launch_sh_t<double>(lmax, E, vec, y, st) : launch_sh_t<float>(lmax, E, vec, y, st);
}

// ------------------------------------------------------------------------------------------
// transpose

__global__ void __launch_bounds__(256) fill_zero(int32_t *a, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) a[i] = 0;
}

__global__ void __launch_bounds__(256) iota(int32_t *a, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) a[i] = (int32_t)i;
}

// count(s) lands at index s + 2 so that the inclusive scan leaves start(s) at s + 1
__global__ void __launch_bounds__(256) count_senders(const int32_t *__restrict__ col, int64_t E, int64_t N,
                                                     int32_t *t_row_ptr)
{
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= E) return;
    const int32_t s = col[e];
    if (s >= 0 && s + 2 <= N) atomicAdd(&t_row_ptr[s + 2], 1);
}

// single-workgroup inclusive scan in place (once per graph, N + 1 entries)
__global__ void __launch_bounds__(1024) scan_inclusive(int32_t *a, int64_t n)
{
    __shared__ int32_t part[1024];
    const int tid = threadIdx.x;
    const int64_t chunk = (n + 1023) / 1024;
    const int64_t lo = tid * chunk, hi = lo + chunk < n ? lo + chunk : n;
    int32_t sum = 0;
    for (int64_t i = lo; i < hi; ++i) sum += a[i];
    part[tid] = sum;
    __syncthreads();
    for (int off = 1; off < 1024; off *= 2) {
        int32_t v = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int32_t run = tid > 0 ? part[tid - 1] : 0;
    for (int64_t i = lo; i < hi; ++i) {
        run += a[i];
        a[i] = run;
    }
}

__global__ void __launch_bounds__(256) place_edges(const int32_t *__restrict__ col, int64_t E, int64_t N,
                                                   int32_t *t_row_ptr, int32_t *t_edge)
{
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= E) return;
    const int32_t s = col[e];
    if (s < 0 || s >= N) return;
    const int32_t pos = atomicAdd(&t_row_ptr[s + 1], 1);
    t_edge[pos] = (int32_t)e;
}

__device__ void sift_down(int32_t *a, int64_t root, int64_t n)
{
    for (;;) {
        int64_t c = 2 * root + 1;
        if (c >= n) return;
        if (c + 1 < n && a[c + 1] > a[c]) ++c;
        if (a[root] >= a[c]) return;
        int32_t t = a[root];
        a[root] = a[c];
        a[c] = t;
        root = c;
    }
}

// ascending edge ids inside every sender segment (makes the order unique)
__global__ void __launch_bounds__(256) sort_segments(const int32_t *__restrict__ t_row_ptr, int64_t N,
                                                     int32_t *t_edge)
{
    const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= N) return;
    int32_t *a = t_edge + t_row_ptr[s];
    const int64_t n = (int64_t)t_row_ptr[s + 1] - t_row_ptr[s];
    if (n <= 32) {
        for (int64_t i = 1; i < n; ++i) {
            int32_t v = a[i];
            int64_t j = i - 1;
            while (j >= 0 && a[j] > v) {
                a[j + 1] = a[j];
                --j;
            }
            a[j + 1] = v;
        }
        return;
    }
    for (int64_t i = n / 2 - 1; i >= 0; --i) sift_down(a, i, n);
    for (int64_t end = n - 1; end > 0; --end) {
        int32_t t = a[0];
        a[0] = a[end];
        a[end] = t;
        sift_down(a, 0, end);
    }
}

// receiver of each transposed edge: binary search in the receiver CSR
__global__ void __launch_bounds__(256) edge_receivers(const int32_t *__restrict__ row_ptr, int64_t N,
                                                      const int32_t *__restrict__ t_edge, int64_t E,
                                                      int32_t *t_dst)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= E) return;
    const int32_t e = t_edge[t];
    int64_t lo = 0, hi = N;  // find n with row_ptr[n] <= e < row_ptr[n + 1]
    while (hi - lo > 1) {
        int64_t mid = (lo + hi) / 2;
        if (row_ptr[mid] <= e) lo = mid;
        else hi = mid;
    }
    t_dst[t] = (int32_t)lo;
}

// ------------------------------------------------------------------------------------------
// heavy-first receiver order: stable bucket sort by floor(log2(degree + 1)), descending

__device__ __forceinline__ int degree_bucket(const int32_t *row_ptr, int64_t i)
{
    const int32_t d = row_ptr[i + 1] - row_ptr[i];
    return 31 - __clz(d + 1);  // floor(log2(d + 1)), 0..31
}

__global__ void __launch_bounds__(1024) degree_order(const int32_t *__restrict__ row_ptr, int64_t N,
                                                     int32_t *__restrict__ order)
{
    __shared__ int32_t cnt[32];
    __shared__ int32_t base[32];
    __shared__ int32_t wcnt[16][32];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    if (tid < 32) cnt[tid] = 0;
    __syncthreads();
    for (int64_t i = tid; i < N; i += 1024) atomicAdd(&cnt[degree_bucket(row_ptr, i)], 1);
    __syncthreads();
    if (tid == 0) {
        int32_t run = 0;
        for (int b = 31; b >= 0; --b) {
            base[b] = run;
            run += cnt[b];
        }
    }
    __syncthreads();
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int64_t c0 = 0; c0 < N; c0 += 1024) {
        const int64_t i = c0 + tid;
        const int b = i < N ? degree_bucket(row_ptr, i) : -1;
        int rank = 0;
        for (int bb = 0; bb < 32; ++bb) {
            const unsigned long long m = __ballot(b == bb);
            if (b == bb) rank = __popcll(m & below);
            if (lane == 0) wcnt[wave][bb] = __popcll(m);
        }
        __syncthreads();
        if (tid < 32) {
            int32_t run = base[tid];
            for (int w = 0; w < 16; ++w) {
                const int32_t t = wcnt[w][tid];
                wcnt[w][tid] = run;
                run += t;
            }
            base[tid] = run;
        }
        __syncthreads();
        if (b >= 0) order[wcnt[wave][b] + rank] = (int32_t)i;
        __syncthreads();
    }
}

hipError_t launch_degree_order(int64_t N, const int32_t *row_ptr, int32_t *order, hipStream_t st)
{
    if (N == 0) return hipSuccess;
    hipLaunchKernelGGL(degree_order, dim3(1), dim3(1024), 0, st, row_ptr, N, order);
    return hipGetLastError();
}

hipError_t launch_transpose(int64_t N, int64_t E, const int32_t *row_ptr, const int32_t *col, int32_t *t_row_ptr,
                            int32_t *t_edge, int32_t *t_dst, hipStream_t st)
{
    auto blocks = [](int64_t n) { return dim3((unsigned)((n + 255) / 256)); };
    hipLaunchKernelGGL(fill_zero, blocks(N + 1), dim3(256), 0, st, t_row_ptr, N + 1);
    if (E > 0) {
        hipLaunchKernelGGL(count_senders, blocks(E), dim3(256), 0, st, col, E, N, t_row_ptr);
        hipLaunchKernelGGL(scan_inclusive, dim3(1), dim3(1024), 0, st, t_row_ptr, N + 1);
        hipLaunchKernelGGL(place_edges, blocks(E), dim3(256), 0, st, col, E, N, t_row_ptr, t_edge);
        if (N > 0) hipLaunchKernelGGL(sort_segments, blocks(N), dim3(256), 0, st, t_row_ptr, N, t_edge);
        hipLaunchKernelGGL(edge_receivers, blocks(E), dim3(256), 0, st, row_ptr, N, t_edge, E, t_dst);
    }
    return hipGetLastError();
}

hipError_t launch_iota(int64_t n, int32_t *a, hipStream_t st)
{
    if (n > 0) hipLaunchKernelGGL(iota, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a, n);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// radial projection of the uvw convolution, one radial channel r at a time (Sobek page,
// Abstract: W_e = rho_e Theta reassociated with the coupling, so that per-edge W blocks are never
// formed).  The coupling is linear in Y, so channel r's share of the convolution is the
// shared-weight convolution of rho[:, r] * Y with Theta's row r.

// ys[e][j] = y[e][j] * rho[e][r]
template <typename T>
__global__ void __launch_bounds__(256) radial_scale_rows(int64_t E, int D, int R, int r, const T *__restrict__ y,
                                                         const T *__restrict__ rho, T *__restrict__ ys)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= E * D) return;
    ys[i] = y[i] * rho[(i / D) * R + r];
}

// With t[e] the gradient of channel r's convolution with respect to its scaled SH row:
// gy[e] (+)= rho[e][r] t[e] (the chain rule through ys = rho y; `acc` 0 writes), grho[e][r] =
// sum_j y[e][j] t[e][j] (j ascending), then t[e] = 0 for the next channel's accumulation.
// A workgroup takes 64 consecutive edges: their rows of t and y are contiguous (64 D values), so
// they are staged through LDS with consecutive threads on consecutive words, and the per-edge dot
// products read them from there.
template <typename T>
__global__ void __launch_bounds__(256) radial_fold_rows(int64_t E, int D, int R, int r, const T *__restrict__ y,
                                                        const T *__restrict__ rho, T *__restrict__ t,
                                                        T *__restrict__ gy, T *__restrict__ grho, int acc)
{
    extern __shared__ __align__(16) unsigned char fold_lds[];
    T *ts = reinterpret_cast<T *>(fold_lds);  // [64 * D]
    T *yl = ts + 64 * D;                       // [64 * D]
    const int64_t e0 = (int64_t)blockIdx.x * 64;
    const int ne = (int)(E - e0 < 64 ? E - e0 : 64);
    const int n = ne * D;
    const int64_t base = e0 * D;
    for (int i = threadIdx.x; i < n; i += 256) {
        ts[i] = t[base + i];
        yl[i] = y[base + i];
    }
    __syncthreads();
    if (grho && (int)threadIdx.x < ne) {
        T d = 0;
        for (int j = 0; j < D; ++j) d += yl[threadIdx.x * D + j] * ts[threadIdx.x * D + j];
        grho[(e0 + threadIdx.x) * R + r] = d;
    }
    for (int i = threadIdx.x; i < n; i += 256) {
        const T s = rho[(e0 + i / D) * R + r];
        if (gy) gy[base + i] = acc ? gy[base + i] + s * ts[i] : s * ts[i];
        t[base + i] = 0;
    }
}

hipError_t launch_radial_scale(bool f64, int64_t E, int D, int R, int r, const void *y, const void *rho, void *ys,
                               hipStream_t st)
{
    const int64_t n = E * D;
    if (n == 0) return hipSuccess;
    const dim3 grid((unsigned)((n + 255) / 256));
    if (f64)
        hipLaunchKernelGGL(radial_scale_rows<double>, grid, dim3(256), 0, st, E, D, R, r, (const double *)y,
                           (const double *)rho, (double *)ys);
    else
        hipLaunchKernelGGL(radial_scale_rows<float>, grid, dim3(256), 0, st, E, D, R, r, (const float *)y,
                           (const float *)rho, (float *)ys);
    return hipGetLastError();
}

hipError_t launch_radial_fold(bool f64, int64_t E, int D, int R, int r, const void *y, const void *rho, void *t,
                              void *gy, void *grho, int acc, hipStream_t st)
{
    if (E == 0) return hipSuccess;
    if (D < 1 || D > 64) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((E + 63) / 64));
    const size_t lds = 2 * 64 * (size_t)D * (f64 ? 8 : 4);  // at most 64 KB
    if (f64)
        hipLaunchKernelGGL(radial_fold_rows<double>, grid, dim3(256), lds, st, E, D, R, r, (const double *)y,
                           (const double *)rho, (double *)t, (double *)gy, (double *)grho, acc);
    else
        hipLaunchKernelGGL(radial_fold_rows<float>, grid, dim3(256), lds, st, E, D, R, r, (const float *)y,
                           (const float *)rho, (float *)t, (float *)gy, (float *)grho, acc);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// scratch of the allocation-free entry point (cgtp_tp_backward_noalloc): a file-scope device
// array, so the library never has to allocate device memory for it.  In host code `scratch` is
// only a handle for the runtime, never a device address: the device address is looked up once
// per device and only that address is handed to kernels.

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_for_current_device(void **ptr)
{
    static std::mutex mu;
    static std::map<int, void *> by_device;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    auto it = by_device.find(dev);
    if (it == by_device.end()) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        it = by_device.emplace(dev, p).first;
    }
    *ptr = it->second;
    return hipSuccess;
}

}  // namespace cgtp
