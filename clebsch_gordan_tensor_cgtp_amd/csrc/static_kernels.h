// Launchers of the fixed kernels of libcgtp (static_kernels.hip).
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>

namespace cgtp {

hipError_t launch_spherical_harmonics(int lmax, bool f64, int64_t E, const void *vec, void *y, hipStream_t st);
hipError_t launch_degree_order(int64_t N, const int32_t *row_ptr, int32_t *order, hipStream_t st);
hipError_t launch_transpose(int64_t N, int64_t E, const int32_t *row_ptr, const int32_t *col, int32_t *t_row_ptr,
                            int32_t *t_edge, int32_t *t_dst, hipStream_t st);
// a[i] = i for i < n
hipError_t launch_iota(int64_t n, int32_t *a, hipStream_t st);
// uvw radial projection, radial channel r of R: ys = rho[:, r] * y (E x D rows), and the fold of
// that channel's SH-row gradient t into grad_y (acc 0 writes) and grad_rho[:, r] (either may be
// NULL), clearing t
hipError_t launch_radial_scale(bool f64, int64_t E, int D, int R, int r, const void *y, const void *rho, void *ys,
                               hipStream_t st);
hipError_t launch_radial_fold(bool f64, int64_t E, int D, int R, int r, const void *y, const void *rho, void *t,
                              void *gy, void *grho, int acc, hipStream_t st);

// Device scratch of the allocation-free entry point: a fixed array of this module, one copy per
// device.  The first call on a device looks its address up (with that device current) and keeps
// it; later calls return the kept address.  Every caller on one device shares the same memory.
constexpr size_t kScratchBytes = size_t(64) << 20;
hipError_t scratch_for_current_device(void **ptr);

}  // namespace cgtp
