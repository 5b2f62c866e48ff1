// Internal launchers of the gfx950 kernels (not part of the public C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

// Payload element type codes (mx_elem_type): 0 = E4M3, 1 = E5M2.

// 1x32 quantisation of a flat BF16 array of n elements (n % 32 == 0).
hipError_t launch_quant_row(const void* x, int64_t n, void* q, void* s, int elem,
                            hipStream_t stream);

// mode 1 = column (q_t, s_t), 2 = dual (q, s, q_t, s_t), 3 = 32x32 tiles (q, s,
// batch 1 only: a stack of tiled matrices is one taller matrix);
// `batch` contiguous [R, C] matrices with contiguous outputs (grid.z).
hipError_t launch_quant_tile(int mode, const void* x, int64_t R, int64_t C, void* q, void* s,
                             void* qt, void* st, int64_t batch, int elem, hipStream_t stream);

// Column blocks restarting at every group offset along the token axis of
// x [T, C]; q_t [C, cap], s_t [C, cap/32] with cap = 128 (T / 128 + G).
hipError_t launch_quant_grouped_col(const void* x, int64_t T, int64_t C, int64_t G,
                                    const int64_t* offsets, int64_t cap, void* qt, void* st,
                                    int elem, hipStream_t stream);

// B operand layouts of the GEMM.
enum GemmB {
  GEMM_B_ROW = 0,     // b [N][K], sb [N][K/32]
  GEMM_B_TILE = 1,    // b [N][K], sb tiles [N/32][K/32]
  GEMM_B_TILE_T = 2,  // b [K][N] contracted over its rows, sb tiles [K/32][N/32]
};

// a_elem / b_elem: payload element types of A and B; num_cus: compute units
// of the device (the persistent grid of the 1x32 GEMM).
hipError_t launch_gemm(int bmode, int a_elem, int b_elem, int64_t M, int64_t N, int64_t K,
                       const void* a, const void* sa, const void* b, const void* sb, void* c,
                       int num_cus, hipStream_t stream);

// The same GEMM (E4M3 operands) with its BF16 result quantised in 1x32
// blocks along N (out_elem 0 = E4M3, 1 = E5M2): q [M, N], s [M, N/32].
hipError_t launch_gemm_q(int bmode, int out_elem, int64_t M, int64_t N, int64_t K, const void* a,
                         const void* sa, const void* b, const void* sb, void* q, void* s,
                         int num_cus, hipStream_t stream);

// a_elem / b_elem: payload element types of the token rows and the expert
// weights.
hipError_t launch_grouped_gemm(int a_elem, int b_elem, int64_t G, const int64_t* offsets, int64_t T,
                               int64_t N, int64_t K, const void* a, const void* sa, const void* b,
                               const void* sb, void* c, int num_cus, hipStream_t stream);

// Per-expert weight gradient c[g] [M, N] over group g's token columns of
// a [M, cap] and b [N, cap] (grouped column layout above).
// num_cus: compute units of the device (the persistent grid has at most one
// workgroup per compute unit).
hipError_t launch_grouped_wgrad(int a_elem, int b_elem, int64_t G, const int64_t* offsets, int64_t T,
                                int64_t M, int64_t N, int64_t cap, const void* a, const void* sa,
                                const void* b, const void* sb, void* c, int num_cus,
                                hipStream_t stream);

// Zero `nbytes` bytes at p (any alignment), as a kernel (no hipMemsetAsync,
// so the call can sit in a captured graph).
hipError_t launch_fill_zero(void* p, int64_t nbytes, hipStream_t stream);

}  // namespace mx
