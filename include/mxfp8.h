/*
 * mxfp8.h -- C ABI of the MXFP8 microscaled-precision hot path on MI355X
 * (gfx950): dynamic MX quantisation of BF16 tensors and the MXFP8 GEMMs that
 * consume the quantised operands and restore a BF16 result.
 *
 * Formats (OCP MX / OFP8, named by the pages, defined by OCP):
 *   BF16   input elements (IEEE binary32 upper half), subnormals honoured.
 *   E4M3   payload byte, bias 7, largest finite 448, 0x7F/0xFF = NaN.
 *   E8M0   scale byte b = 2^(b-127), 0xFF = NaN.
 *
 * Conventions for every call:
 *   - Pointers named x, q, s, q_t, s_t, a, sa, b, sb, c, offsets are DEVICE
 *     pointers owned by the caller; the library never allocates, frees or
 *     retains them beyond the completion of the work it enqueued.
 *   - All work is enqueued asynchronously on `stream` (0 = the null stream)
 *     of the current device; results are visible after the stream syncs.
 *   - Arguments are validated on the host before anything is launched; on a
 *     non-zero status nothing was launched and no output was touched.
 *     Validation errors mirror the ValueError the pages raise for an
 *     unsupported block size or recipe (MindSpeed RFC "add MXFP8-32x32
 *     quantisation support to FSDP", sections 3.4 and 3.5.2.1).
 *   - A shape whose launch grid would reach 2^32 work-items in one
 *     dimension (far beyond any tensor that fits in device memory) returns
 *     MX_ERR_UNSUPPORTED_SHAPE rather than launching a truncated grid.
 *   - The GEMMs address a 256-row tile of an operand with 32-bit byte
 *     offsets, so the contraction length is limited: K < 2^23 for mx_gemm,
 *     mx_gemm_elem, mx_gemm_quant and mx_grouped_gemm(_elem), (K + 256) * N
 *     < 2^31 for the 32x32 dgrad's transposed weight, and 256 * cap < 2^31
 *     for the per-group token capacity of the MoE backward; the grouped
 *     GEMM numbers its 256x256 output tiles with 32-bit indices, so
 *     (ceil(T / 256) + G) * ceil(N / 256) < 2^31.  Beyond that they return
 *     MX_ERR_UNSUPPORTED_SHAPE.
 *   - The current device must be gfx950; otherwise calls return
 *     MX_ERR_UNSUPPORTED_DEVICE (the pages' init-time hardware gate:
 *     torchtitan-npu MXFP8/HiF8 tutorial, "hardware requirement").
 *   - No exception crosses the ABI; the last error detail of the calling
 *     thread is available from mx_last_error().
 */
#ifndef MXFP8_H
#define MXFP8_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mx_status {
    MX_OK = 0,
    MX_ERR_INVALID_ARG = 1,        /* null pointer, negative size, unknown enum value */
    MX_ERR_UNSUPPORTED_SHAPE = 2,  /* a dimension the mode's block size does not divide */
    MX_ERR_UNSUPPORTED_DEVICE = 3, /* the current device is not gfx950 */
    MX_ERR_HIP = 4                 /* a HIP runtime call failed (see mx_last_error) */
} mx_status;

/* Quantisation modes.  "1x32" is the MX block of 32 consecutive elements
 * sharing one E8M0 scale (torchtitan-npu MXFP8/HiF8 tutorial, "MXFP8 / HiF8
 * architecture overview", MXFP8 bullet); dual-axis quantises the same tensor
 * along both axes in one pass (tutorial, step-2 environment table,
 * MXFP8_DUAL_AXIS_FORWARD; RFC section 3.3.3); 32x32 is block size
 * [1,32,32]: one scale per 32x32 weight tile, one FP8 weight shared by
 * forward and backward (RFC sections 1.1, 3.1, 3.3.3). */
typedef enum mx_quant_mode {
    MX_QUANT_ROW_1x32 = 0,   /* blocks of 32 along each row (the last, contiguous dim) */
    MX_QUANT_COL_1x32 = 1,   /* blocks of 32 down each column, written transposed */
    MX_QUANT_DUAL_AXIS = 2,  /* ROW and COL outputs from one read of x */
    MX_QUANT_BLOCK_32x32 = 3 /* one scale per 32x32 tile */
} mx_quant_mode;

/* Payload element type.  E4M3 is the pages' element type for every tensor
 * (RFC section 3.3.1); E5M2 is the other FP8 dst_type the RFC's recipe
 * accepts (section 3.5.2.3).  OCP E5M2: bias 15, largest finite 57344,
 * 0x7C infinity, 0x7D..0x7F NaN.  With E5M2 the scale keeps the rceil rule
 * against 57344: the smallest e with amax <= 57344 * 2^e. */
typedef enum mx_elem_type {
    MX_ELEM_E4M3 = 0,
    MX_ELEM_E5M2 = 1
} mx_elem_type;

/* Which product of a linear layer a GEMM call computes (operand roles).
 * Each is an FP8 matmul over MX-quantised operands whose result is restored
 * to BF16 (torchtitan-npu MXFP8/HiF8 tutorial, "MXFP8 / HiF8 architecture
 * overview", MXFP8 bullet); the forward product takes the operands blocked
 * along the contraction, the backward products the copies blocked along the
 * other axis (tutorial, step-2 environment table, MXFP8_DUAL_AXIS_FORWARD;
 * MindSpeed RFC "add MXFP8-32x32 quantisation support to FSDP", section
 * 3.3.3: weight_fwd / weight_bwd). */
typedef enum mx_gemm_layout {
    MX_GEMM_FPROP = 0, /* Y  = X  * W^T : a = X rows,     b = W rows            */
    MX_GEMM_DGRAD = 1, /* dX = dY * W   : a = dY rows,    b = W columns (W_col_T) */
    MX_GEMM_WGRAD = 2  /* dW = dY^T * X : a = dY columns, b = X columns          */
} mx_gemm_layout;

/* Granularity of the B operand's scales. */
typedef enum mx_bscale_kind {
    MX_BSCALE_1x32 = 0, /* one scale per 32 K-elements of each B row */
    MX_BSCALE_32x32 = 1 /* one scale per 32x32 tile of a 32x32-quantised weight */
} mx_bscale_kind;

/* MX_OK iff `device` is a gfx950 GPU.  MX_ERR_UNSUPPORTED_DEVICE for another
 * architecture, MX_ERR_HIP if the device cannot be queried. */
mx_status mx_device_check(int device);

/* 1 iff a HIP architecture name (e.g. "gfx950:sramecc+:xnack-") denotes a
 * device this library runs on.  Pure host function, no HIP call. */
int mx_arch_supported(const char* gcn_arch_name);

/* Static description of a status code.  Never NULL. */
const char* mx_status_string(mx_status s);

/* Detail of the last failing call on this thread ("" if none).  Never NULL;
 * valid until the next call on this thread. */
const char* mx_last_error(void);

/* Dynamic MX quantisation of x, BF16 [rows, cols] row-major, to E4M3 payload
 * bytes and E8M0 scale bytes.  The scale exponent of a block is the smallest
 * e with amax <= 448 * 2^e (the "rceil" rule), clamped to [-127, 127]; each
 * element is divided by 2^e and rounded to nearest-even into E4M3 (the
 * tutorial's step-3 log names the recipe mxfp8_rceil; RFC section 3.3.1 fixes
 * the element type to E4M3).  An all-zero block gets scale 0x00; a block
 * holding NaN or Inf gets scale 0xFF and payload 0x7F.
 *
 * Outputs by mode (all row-major, uint8):
 *   ROW_1x32:    q [rows, cols],  s [rows, cols/32]          needs cols % 32 == 0
 *   COL_1x32:    q_t [cols, rows], s_t [cols, rows/32]       needs both % 32 == 0
 *                (q_t[c][r] quantises x[r][c] with the block x[32i..32i+31][c])
 *   DUAL_AXIS:   q, s, q_t, s_t as above, one read of x      needs both % 32 == 0
 *   BLOCK_32x32: q [rows, cols], s [rows/32, cols/32]        needs both % 32 == 0
 *                (s is both the forward and the backward scale: the forward
 *                 view blocks K along cols, the backward view along rows)
 * Unused output pointers may be NULL.  rows == 0 or cols == 0 is a no-op. */
mx_status mx_quant(mx_quant_mode mode, const void* x, int64_t rows, int64_t cols, void* q, void* s,
                   void* q_t, void* s_t, hipStream_t stream);

/* mx_quant with a choice of payload element type (E4M3 or E5M2); every
 * other rule, layout and shape requirement is that of mx_quant, which is
 * mx_quant_elem with MX_ELEM_E4M3.  A NaN/Inf block gets scale 0xFF and
 * payload 0x7F in both types. */
mx_status mx_quant_elem(mx_quant_mode mode, mx_elem_type elem, const void* x, int64_t rows,
                        int64_t cols, void* q, void* s, void* q_t, void* s_t, hipStream_t stream);

/* MXFP8 GEMM C = A * B^T with FP32 accumulation and a BF16 result: the
 * FP8 matmul of MX-quantised operands whose output is restored to BF16
 * (torchtitan-npu MXFP8/HiF8 tutorial, "MXFP8 / HiF8 architecture
 * overview", MXFP8 bullet); with 32x32 weight scales, forward and backward
 * share one FP8 weight and differ only in the scale view (MindSpeed RFC "add
 * MXFP8-32x32 quantisation support to FSDP", sections 3.1 and 3.3.3).
 *   a:  E4M3 [M, K] row-major, sa: E8M0 [M, K/32]
 *   b/sb by (layout, bkind):
 *     any layout, MX_BSCALE_1x32:   b [N, K], sb [N, K/32]      ("TN": both K-contiguous)
 *     MX_GEMM_FPROP, MX_BSCALE_32x32: b [N, K], sb tiles [N/32, K/32]
 *     MX_GEMM_DGRAD, MX_BSCALE_32x32: b [K, N] -- the one shared FP8 weight
 *         [out = K, in = N] -- contracted over its rows, sb tiles [K/32, N/32]
 *     MX_GEMM_WGRAD, MX_BSCALE_32x32: invalid (the weight-gradient product
 *         has no weight operand)
 *   c:  BF16 [M, N] row-major.
 * C[m][n] = sum_k E4M3(a[m][k]) 2^(sa[m][k/32]-127) * E4M3(B[n][k]) 2^(sB-127).
 * Requires K % 32 == 0 (and N % 32 == 0 for 32x32 scales).  K == 0 writes
 * zeros (a, sa, b, sb are then not read and may be NULL); M == 0 or N == 0
 * is a no-op.  Errors: MX_ERR_INVALID_ARG for an unknown enum value, a
 * negative size or a NULL pointer that would be read or written;
 * MX_ERR_UNSUPPORTED_SHAPE for the divisibility and size rules above. */
mx_status mx_gemm(mx_gemm_layout layout, mx_bscale_kind bkind, int64_t M, int64_t N, int64_t K,
                  const void* a, const void* sa, const void* b, const void* sb, void* c,
                  hipStream_t stream);

/* mx_gemm with the payload element type of each operand (E4M3 or E5M2, in
 * any combination, e.g. E5M2 gradients against an E4M3 weight); layouts,
 * scales and rules as mx_gemm, which is mx_gemm_elem with E4M3 operands. */
mx_status mx_gemm_elem(mx_gemm_layout layout, mx_bscale_kind bkind, mx_elem_type a_elem,
                       mx_elem_type b_elem, int64_t M, int64_t N, int64_t K, const void* a,
                       const void* sa, const void* b, const void* sb, void* c, hipStream_t stream);

/* Fused producer: mx_gemm (E4M3 operands) whose BF16 result is quantised
 * in the epilogue, in 1x32 blocks along N, instead of being written: the
 * next GEMM's row-quantised operand straight from this one, without the
 * BF16 round trip through memory (the pages stress fusing the memory-bound
 * steps around the matmuls: torchtitan-npu practice page, AutoFuse).
 *   q: [M, N] payload of out_elem (E4M3 or E5M2), s: E8M0 [M, N/32];
 *   the bytes equal mx_quant_elem(MX_QUANT_ROW_1x32, out_elem) applied to
 *   the BF16 result mx_gemm would write (same rounding to BF16, same rule).
 * Layouts and operand rules as mx_gemm; requires N % 32 == 0 as well.
 * M == 0 or N == 0 is a no-op; K == 0 writes zero payload and scales
 * (0x00 bytes: an all-zero block) without reading a, sa, b or sb. */
mx_status mx_gemm_quant(mx_gemm_layout layout, mx_bscale_kind bkind, mx_elem_type out_elem,
                        int64_t M, int64_t N, int64_t K, const void* a, const void* sa,
                        const void* b, const void* sb, void* q, void* s, hipStream_t stream);

/* MoE grouped MXFP8 GEMM over per-expert token groups (tutorial, "MXFP8 /
 * HiF8 architecture overview": MoE expert layers run as grouped matmul; RFC
 * section 2.2, gate_up_proj / down_proj).
 *   offsets: DEVICE int64 [G+1], offsets[0] = 0, offsets[G] = T,
 *            non-decreasing; rows offsets[g] .. offsets[g+1]-1 of a belong
 *            to expert g (groups may be empty, sizes need not be multiples
 *            of 32).  Offsets are read on the device and trusted; values
 *            outside [0, T] are clamped and a decrease is treated as an empty
 *            group, so bad offsets give wrong rows but never a bad access.
 *   a: E4M3 [T, K], sa [T, K/32];  b: E4M3 [G, N, K], sb [G, N, K/32]
 *   c: BF16 [T, N]; row r of expert g is  c[r] = a[r] * b[g]^T.
 *   workspace: DEVICE scratch of at least
 *            mx_grouped_gemm_workspace_size(G, T, N) bytes, owned by the
 *            caller (may be NULL when that size is 0, as it is in this
 *            version: the kernel derives its tile list from the offsets on
 *            the device, so it is not touched).
 * Requires K % 32 == 0 and 1 <= G <= 512.  T == 0 or N == 0 is a no-op.
 * Errors: MX_ERR_INVALID_ARG for G outside [1, 512], a negative size, a NULL
 * pointer that would be read or written, or workspace_bytes below the
 * required size; MX_ERR_UNSUPPORTED_SHAPE for K % 32 != 0 or K too large. */
mx_status mx_grouped_gemm(int64_t G, const int64_t* offsets, int64_t T, int64_t N, int64_t K,
                          const void* a, const void* sa, const void* b, const void* sb, void* c,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace mx_grouped_gemm and mx_grouped_gemm_elem need
 * for G groups, T token rows and N output columns.  Pure host function, no
 * HIP call; currently 0 for every shape. */
size_t mx_grouped_gemm_workspace_size(int64_t G, int64_t T, int64_t N);

/* mx_grouped_gemm with the payload element type of each operand chosen
 * (E4M3 or E5M2, the RFC's two FP8 dst_types, section 3.5.2.3): a_elem for
 * the token rows a (e.g. E5M2 gradients in the MoE backward-data product),
 * b_elem for the expert weights b.  Scales, layouts, rules and errors as
 * mx_grouped_gemm, which is this call with E4M3 for both (the workspace
 * rule included); an unknown element type returns MX_ERR_INVALID_ARG. */
mx_status mx_grouped_gemm_elem(mx_elem_type a_elem, mx_elem_type b_elem, int64_t G,
                               const int64_t* offsets, int64_t T, int64_t N, int64_t K,
                               const void* a, const void* sa, const void* b, const void* sb,
                               void* c, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* mx_quant over a batch of equally shaped matrices, e.g. the per-expert
 * weights [G, rows, cols] of an MoE layer (the RFC quantises gate_up_proj /
 * down_proj of every expert, section 2.2).  x holds `batch` contiguous BF16
 * [rows, cols] matrices; every output is the stack of the per-matrix outputs
 * of mx_quant in the same mode (q [batch, rows, cols], s [batch, rows,
 * cols/32], q_t [batch, cols, rows], s_t [batch, cols, rows/32]; 32x32 tiles
 * s [batch, rows/32, cols/32]).  Shape rules as mx_quant; 1 <= batch <= 65535.
 * batch == 0 is a no-op. */
mx_status mx_quant_batched(mx_quant_mode mode, const void* x, int64_t batch, int64_t rows,
                           int64_t cols, void* q, void* s, void* q_t, void* s_t,
                           hipStream_t stream);

/* mx_quant_batched with the payload element type chosen (E4M3 or E5M2, the
 * RFC's two FP8 dst_types, section 3.5.2.3), with the scale rule for that
 * type as in mx_quant_elem.  Shapes, layouts and errors as mx_quant_batched,
 * which is this call with E4M3; an unknown element type returns
 * MX_ERR_INVALID_ARG. */
mx_status mx_quant_batched_elem(mx_quant_mode mode, mx_elem_type elem, const void* x,
                                int64_t batch, int64_t rows, int64_t cols, void* q, void* s,
                                void* q_t, void* s_t, hipStream_t stream);

/* Columns of the per-group column-quantised token matrix: 128 * (T / 128 + G)
 * (integer division).  Returns -1 for T < 0 or G < 1. */
int64_t mx_grouped_col_capacity(int64_t T, int64_t G);

/* MoE backward quantisation of a token matrix along the token axis, per
 * expert group (RFC section 2.2: grouped-matmul quantisation of the MoE
 * experts; the backward weight-gradient product contracts over each group's
 * tokens).  x: BF16 [T, C] with the groups' rows in order; offsets: DEVICE
 * int64 [G+1] as in mx_grouped_gemm.  Blocks of 32 tokens restart at every
 * group offset; the last block of a group holds only its remaining tokens and
 * its amax covers those alone.  Output, transposed like the column mode:
 *   q_t [C, cap], s_t [C, cap / 32], cap = mx_grouped_col_capacity(T, G);
 *   token o_g + k of group g sits at column P_g + k, P_g = 128 (o_g / 128 + g);
 *   every column holding no token is part of an all-zero block (payload
 *   0x00, scale 0x00), so each group's range [P_g, P_g + 128 ceil(m_g / 128))
 *   is zero past its tokens.
 * Requires C % 32 == 0, 1 <= G <= 512, 256 * cap < 2^31.  Offsets are read
 * on the device and clamped into [0, T]; bad offsets give wrong blocks but
 * never a bad access.  x may be NULL when T == 0 (the outputs are then all
 * zero blocks).  C == 0 is a no-op. */
mx_status mx_quant_grouped_col(const void* x, int64_t T, int64_t C, int64_t G,
                               const int64_t* offsets, void* q_t, void* s_t, hipStream_t stream);

/* mx_quant_grouped_col with the payload element type chosen (E4M3 or E5M2,
 * the RFC's two FP8 dst_types, section 3.5.2.3; e.g. E5M2 gradients for the
 * weight-gradient product).  The scale rule is rceil against the type's
 * largest finite value, as in mx_quant_elem; layout, rules and errors as
 * mx_quant_grouped_col (which is this call with E4M3); an unknown element
 * type returns MX_ERR_INVALID_ARG. */
mx_status mx_quant_grouped_col_elem(mx_elem_type elem, const void* x, int64_t T, int64_t C,
                                    int64_t G, const int64_t* offsets, void* q_t, void* s_t,
                                    hipStream_t stream);

/* Per-expert weight gradient of the MoE backward (RFC section 2.2):
 *   c[g][m][n] = sum over the tokens t of group g of dY[t][m] * X[t][n]
 * from the grouped column quantisations a = (q_t, s_t) of dY [T, M] and
 * b = (q_t, s_t) of X [T, N] (mx_quant_grouped_col with the same offsets):
 *   a [M, cap] + sa [M, cap/32], b [N, cap] + sb [N, cap/32],
 *   c: BF16 [G, M, N]; an empty group gets zeros.
 * FP32 accumulation, BF16 result; the columns of a group's range past its
 * tokens must hold zero payload (as mx_quant_grouped_col writes them).
 * Requires 1 <= G <= 512, 256 * cap < 2^31.  M == 0 or N == 0 is a no-op. */
mx_status mx_grouped_gemm_wgrad(int64_t G, const int64_t* offsets, int64_t T, int64_t M, int64_t N,
                                const void* a, const void* sa, const void* b, const void* sb,
                                void* c, hipStream_t stream);

/* mx_grouped_gemm_wgrad with the payload element type of each operand
 * chosen: a_elem for a (the gradient), b_elem for b (the input), each E4M3
 * or E5M2 as its mx_quant_grouped_col_elem call wrote it.  Rules and errors
 * as mx_grouped_gemm_wgrad (which is this call with E4M3 for both); an
 * unknown element type returns MX_ERR_INVALID_ARG. */
mx_status mx_grouped_gemm_wgrad_elem(mx_elem_type a_elem, mx_elem_type b_elem, int64_t G,
                                     const int64_t* offsets, int64_t T, int64_t M, int64_t N,
                                     const void* a, const void* sa, const void* b, const void* sb,
                                     void* c, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MXFP8_H */
