// Host side of the C ABI declared in include/mxfp8.h: argument validation
// (before any HIP call), the gfx950 gate, and dispatch to the kernels.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/mxfp8.h"
#include "mx_kernels.h"

namespace {

thread_local char g_err[512] = "";

mx_status fail(mx_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

mx_status hip_fail(hipError_t e, const char* what) {
  return fail(MX_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
int g_arch_ok[MAX_DEVICES];  // 0 unknown, 1 gfx950, 2 other
int g_num_cus[MAX_DEVICES];

mx_status check_device(int dev) {
  if (dev < 0 || dev >= MAX_DEVICES) return fail(MX_ERR_INVALID_ARG, "device %d out of range", dev);
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_arch_ok[dev] == 1) return MX_OK;
    if (g_arch_ok[dev] == 2)
      return fail(MX_ERR_UNSUPPORTED_DEVICE, "MXFP8 kernels need a gfx950 (MI355X) device");
  }
  hipDeviceProp_t prop;
  hipError_t e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
  const bool ok = mx_arch_supported(prop.gcnArchName) != 0;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    g_arch_ok[dev] = ok ? 1 : 2;
    g_num_cus[dev] = prop.multiProcessorCount;
  }
  if (!ok)
    return fail(MX_ERR_UNSUPPORTED_DEVICE, "MXFP8 kernels need a gfx950 (MI355X) device, found %s",
                prop.gcnArchName);
  return MX_OK;
}

mx_status current_device(int* dev) {
  hipError_t e = hipGetDevice(dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  return check_device(*dev);
}

bool mul_overflows(int64_t a, int64_t b) { return a != 0 && b > INT64_MAX / a; }

// A launch grid holds fewer than 2^32 work-items per dimension: `tiles`
// workgroups of 256 threads (one per 256 x 256 output tile).
bool grid_too_large(int64_t tiles) { return tiles >= (int64_t(1) << 32) / 256; }

int64_t gemm_tiles(int64_t M, int64_t N) { return ((M + 255) / 256) * ((N + 255) / 256); }

// The 2-D quantisation grid: one 512-thread workgroup per 128-row tile in x.
bool row_tiles_too_large(int64_t R) { return ((R + 127) / 128) * 512 >= (int64_t(1) << 32); }

// The GEMM kernels address a 256-row tile with 32-bit offsets (rows * K or
// rows * cap bytes, out-of-range loads flagged by bit 31).
constexpr int64_t K_LIMIT = (int64_t(1) << 31) / 256;

}  // namespace

extern "C" {

int mx_arch_supported(const char* name) {
  if (!name) return 0;
  // "gfx950" optionally followed by target features (":sramecc+:xnack-")
  return std::strncmp(name, "gfx950", 6) == 0 && (name[6] == '\0' || name[6] == ':');
}

const char* mx_status_string(mx_status s) {
  switch (s) {
    case MX_OK: return "success";
    case MX_ERR_INVALID_ARG: return "invalid argument";
    case MX_ERR_UNSUPPORTED_SHAPE: return "unsupported shape for the MX block size";
    case MX_ERR_UNSUPPORTED_DEVICE: return "MXFP8 is only supported on gfx950 (MI355X)";
    case MX_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* mx_last_error(void) { return g_err; }

mx_status mx_device_check(int device) {
  g_err[0] = '\0';
  int n = 0;
  hipError_t e = hipGetDeviceCount(&n);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceCount");
  if (device < 0 || device >= n) return fail(MX_ERR_INVALID_ARG, "no device %d (count %d)", device, n);
  return check_device(device);
}

mx_status mx_quant_elem(mx_quant_mode mode, mx_elem_type elem, const void* x, int64_t rows,
                        int64_t cols, void* q, void* s, void* q_t, void* s_t, hipStream_t stream) {
  g_err[0] = '\0';
  if (mode < MX_QUANT_ROW_1x32 || mode > MX_QUANT_BLOCK_32x32)
    return fail(MX_ERR_INVALID_ARG, "unknown quantisation mode %d", (int)mode);
  if (elem != MX_ELEM_E4M3 && elem != MX_ELEM_E5M2)
    return fail(MX_ERR_INVALID_ARG, "unknown element type %d", (int)elem);
  if (rows < 0 || cols < 0) return fail(MX_ERR_INVALID_ARG, "negative shape [%lld, %lld]",
                                        (long long)rows, (long long)cols);
  if (mul_overflows(rows, cols) || (rows * cols) > (INT64_MAX / 4))
    return fail(MX_ERR_INVALID_ARG, "shape too large");
  const bool need_row = mode == MX_QUANT_ROW_1x32 || mode == MX_QUANT_DUAL_AXIS ||
                        mode == MX_QUANT_BLOCK_32x32;
  const bool need_col = mode == MX_QUANT_COL_1x32 || mode == MX_QUANT_DUAL_AXIS;
  // every mode tiles the columns by 32; all but ROW block or tile the rows by 32
  if (cols % 32 != 0)
    return fail(MX_ERR_UNSUPPORTED_SHAPE, "cols %lld is not a multiple of 32", (long long)cols);
  if (mode != MX_QUANT_ROW_1x32 && rows % 32 != 0)
    return fail(MX_ERR_UNSUPPORTED_SHAPE, "rows %lld is not a multiple of 32", (long long)rows);
  if (mode != MX_QUANT_ROW_1x32 && (cols + 127) / 128 > 65535)
    return fail(MX_ERR_UNSUPPORTED_SHAPE, "cols %lld exceeds the column-tile grid", (long long)cols);
  if (mode != MX_QUANT_ROW_1x32 && row_tiles_too_large(rows))
    return fail(MX_ERR_UNSUPPORTED_SHAPE, "rows %lld exceed the row-tile grid", (long long)rows);
  if (rows == 0 || cols == 0) return MX_OK;
  if (!x) return fail(MX_ERR_INVALID_ARG, "x is NULL");
  if (need_row && (!q || !s)) return fail(MX_ERR_INVALID_ARG, "q and s are required for this mode");
  if (need_col && (!q_t || !s_t))
    return fail(MX_ERR_INVALID_ARG, "q_t and s_t are required for this mode");
  int dev;
  mx_status st = current_device(&dev);
  if (st != MX_OK) return st;
  hipError_t e;
  const int el = (int)elem;
  switch (mode) {
    case MX_QUANT_ROW_1x32: e = mx::launch_quant_row(x, rows * cols, q, s, el, stream); break;
    case MX_QUANT_COL_1x32: e = mx::launch_quant_tile(1, x, rows, cols, q, s, q_t, s_t, 1, el, stream); break;
    case MX_QUANT_DUAL_AXIS: e = mx::launch_quant_tile(2, x, rows, cols, q, s, q_t, s_t, 1, el, stream); break;
    default: e = mx::launch_quant_tile(3, x, rows, cols, q, s, q_t, s_t, 1, el, stream); break;
  }
  if (e != hipSuccess) return hip_fail(e, "quantisation kernel launch");
  return MX_OK;
}

mx_status mx_quant(mx_quant_mode mode, const void* x, int64_t rows, int64_t cols, void* q, void* s,
                   void* q_t, void* s_t, hipStream_t stream) {
  return mx_quant_elem(mode, MX_ELEM_E4M3, x, rows, cols, q, s, q_t, s_t, stream);
}

mx_status mx_gemm_elem(mx_gemm_layout layout, mx_bscale_kind bkind, mx_elem_type a_elem,
                       mx_elem_type b_elem, int64_t M, int64_t N, int64_t K, const void* a,
                       const void* sa, const void* b, const void* sb, void* c, hipStream_t stream) {
  g_err[0] = '\0';
  if ((a_elem != MX_ELEM_E4M3 && a_elem != MX_ELEM_E5M2) ||
      (b_elem != MX_ELEM_E4M3 && b_elem != MX_ELEM_E5M2))
    return fail(MX_ERR_INVALID_ARG, "unknown element type (a %d, b %d)", (int)a_elem, (int)b_elem);
  if (layout < MX_GEMM_FPROP || layout > MX_GEMM_WGRAD)
    return fail(MX_ERR_INVALID_ARG, "unknown GEMM layout %d", (int)layout);
  if (bkind != MX_BSCALE_1x32 && bkind != MX_BSCALE_32x32)
    return fail(MX_ERR_INVALID_ARG, "unknown B scale kind %d", (int)bkind);
  if (bkind == MX_BSCALE_32x32 && layout == MX_GEMM_WGRAD)
    return fail(MX_ERR_INVALID_ARG, "the weight-gradient GEMM has no 32x32 weight operand");
  if (M < 0 || N < 0 || K < 0) return fail(MX_ERR_INVALID_ARG, "negative GEMM shape");
  if (mul_overflows(M, K) || mul_overflows(N, K) || mul_overflows(M, N) || M * N > INT64_MAX / 2)
    return fail(MX_ERR_INVALID_ARG, "GEMM shape too large");
  if (K % 32 != 0) return fail(MX_ERR_UNSUPPORTED_SHAPE, "K %lld is not a multiple of 32", (long long)K);
  if (K >= K_LIMIT)
    return fail(MX_ERR_UNSUPPORTED_SHAPE, "K %lld too large for 32-bit tile offsets", (long long)K);
  if (grid_too_large(gemm_tiles(M, N)))
    return fail(MX_ERR_UNSUPPORTED_SHAPE, "%lld x %lld output tiles exceed one launch grid",
                (long long)M, (long long)N);
  if (bkind == MX_BSCALE_32x32 && layout == MX_GEMM_DGRAD && (K + 256) * N >= (int64_t(1) << 31))
    return fail(MX_ERR_UNSUPPORTED_SHAPE, "transposed 32x32 weight of %lld x %lld bytes too large",
                (long long)K, (long long)N);
  if (bkind == MX_BSCALE_32x32 && N % 32 != 0)
    return fail(MX_ERR_UNSUPPORTED_SHAPE, "N %lld is not a multiple of 32 (32x32 weight tiles)",
                (long long)N);
  if (M == 0 || N == 0) return MX_OK;
  if (!c) return fail(MX_ERR_INVALID_ARG, "c is NULL");
  if (K > 0 && (!a || !sa || !b || !sb)) return fail(MX_ERR_INVALID_ARG, "an operand is NULL");
  int dev;
  mx_status st = current_device(&dev);
  if (st != MX_OK) return st;
  hipError_t e;
  if (K == 0) {
    e = mx::launch_fill_zero(c, 2 * M * N, stream);
  } else {
    int bmode = mx::GEMM_B_ROW;
    if (bkind == MX_BSCALE_32x32) bmode = layout == MX_GEMM_DGRAD ? mx::GEMM_B_TILE_T : mx::GEMM_B_TILE;
    int cus;
    {
      std::lock_guard<std::mutex> lk(g_mu);
      cus = g_num_cus[dev];
    }
    e = mx::launch_gemm(bmode, (int)a_elem, (int)b_elem, M, N, K, a, sa, b, sb, c, cus, stream);
  }
  if (e != hipSuccess) return hip_fail(e, "GEMM kernel launch");
  return MX_OK;
}

mx_status mx_gemm(mx_gemm_layout layout, mx_bscale_kind bkind, int64_t M, int64_t N, int64_t K,
                  const void* a, const void* sa, const void* b, const void* sb, void* c,
                  hipStream_t stream) {
  return mx_gemm_elem(layout, bkind, MX_ELEM_E4M3, MX_ELEM_E4M3, M, N, K, a, sa, b, sb, c, stream);
}

mx_status mx_gemm_quant(mx_gemm_layout layout, mx_bscale_kind bkind, mx_elem_type out_elem,
                        int64_t M, int64_t N, int64_t K, const void* a, const void* sa,
                        const void* b, const void* sb, void* q, void* s, hipStream_t stream) {
  g_err[0] = '\0';
  if (layout < MX_GEMM_FPROP || layout > MX_GEMM_WGRAD)
    return fail(MX_ERR_INVALID_ARG, "unknown GEMM layout %d", (int)layout);
  if (bkind != MX_BSCALE_1x32 && bkind != MX_BSCALE_32x32)
    return fail(MX_ERR_INVALID_ARG, "unknown B scale kind %d", (int)bkind);
  if (out_elem != MX_ELEM_E4M3 && out_elem != MX_ELEM_E5M2)
    return fail(MX_ERR_INVALID_ARG, "unknown element type %d", (int)out_elem);
  if (bkind == MX_BSCALE_32x32 && layout == MX_GEMM_WGRAD)
    return fail(MX_ERR_INVALID_ARG, "the weight-gradient GEMM has no 32x32 weight operand");
  if (M < 0 || N < 0 || K < 0) return fail(MX_ERR_INVALID_ARG, "negative GEMM shape");
  if (mul_overflows(M, K) || mul_overflows(N, K) || mul_overflows(M, N) || M * N > INT64_MAX / 2)
    return fail(MX_ERR_INVALID_ARG, "GEMM shape too large");
  if (K % 32 != 0) return fail(MX_ERR_UNSUPPORTED_SHAPE, "K %lld is not a multiple of 32", (long long)K);
  if (N % 32 != 0)
    return fail(MX_ERR_UNSUPPORTED_SHAPE, "N %lld is not a multiple of 32 (1x32 output blocks)",
                (long long)N);
  if (K >= K_LIMIT)
    return fail(MX_ERR_UNSUPPORTED_SHAPE, "K %lld too large for 32-bit tile offsets", (long long)K);
  if (grid_too_large(gemm_tiles(M, N)))
    return fail(MX_ERR_UNSUPPORTED_SHAPE, "%lld x %lld output tiles exceed one launch grid",
                (long long)M, (long long)N);
  if (bkind == MX_BSCALE_32x32 && layout == MX_GEMM_DGRAD && (K + 256) * N >= (int64_t(1) << 31))
    return fail(MX_ERR_UNSUPPORTED_SHAPE, "transposed 32x32 weight of %lld x %lld bytes too large",
                (long long)K, (long long)N);
  if (M == 0 || N == 0) return MX_OK;
  if (!q || !s) return fail(MX_ERR_INVALID_ARG, "q or s is NULL");
  if (K > 0 && (!a || !sa || !b || !sb)) return fail(MX_ERR_INVALID_ARG, "an operand is NULL");
  int dev;
  mx_status st = current_device(&dev);
  if (st != MX_OK) return st;
  hipError_t e;
  if (K == 0) {
    // an empty contraction: every block of the result is zero (payload 0x00,
    // scale 0x00); no GEMM kernel sees a zero-length operand
    e = mx::launch_fill_zero(q, M * N, stream);
    if (e == hipSuccess) e = mx::launch_fill_zero(s, M * (N / 32), stream);
  } else {
    int bmode = mx::GEMM_B_ROW;
    if (bkind == MX_BSCALE_32x32) bmode = layout == MX_GEMM_DGRAD ? mx::GEMM_B_TILE_T : mx::GEMM_B_TILE;
    int cus;
    {
      std::lock_guard<std::mutex> lk(g_mu);
      cus = g_num_cus[dev];
    }
    e = mx::launch_gemm_q(bmode, (int)out_elem, M, N, K, a, sa, b, sb, q, s, cus, stream);
  }
  if (e != hipSuccess) return hip_fail(e, "fused GEMM kernel launch");
  return MX_OK;
}

size_t mx_grouped_gemm_workspace_size(int64_t G, int64_t T, int64_t N) {
  (void)G;
  (void)T;
  (void)N;
  return 0;  // the persistent kernel derives its tile list from the offsets on the device
}

mx_status mx_grouped_gemm_elem(mx_elem_type a_elem, mx_elem_type b_elem, int64_t G,
                               const int64_t* offsets, int64_t T, int64_t N, int64_t K,
                               const void* a, const void* sa, const void* b, const void* sb,
                               void* c, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  g_err[0] = '\0';
  if ((a_elem != MX_ELEM_E4M3 && a_elem != MX_ELEM_E5M2) ||
      (b_elem != MX_ELEM_E4M3 && b_elem != MX_ELEM_E5M2))
    return fail(MX_ERR_INVALID_ARG, "unknown element type (a %d, b %d)", (int)a_elem, (int)b_elem);
  if (G < 1 || G > 512) return fail(MX_ERR_INVALID_ARG, "group count %lld not in [1, 512]", (long long)G);
  if (T < 0 || N < 0 || K < 0) return fail(MX_ERR_INVALID_ARG, "negative grouped GEMM shape");
  if (mul_overflows(T, K) || mul_overflows(T, N) || mul_overflows(G, N) || mul_overflows(G * N, K) ||
      T * N > INT64_MAX / 2)
    return fail(MX_ERR_INVALID_ARG, "grouped GEMM shape too large");
  const size_t need = mx_grouped_gemm_workspace_size(G, T, N);
  if (workspace_bytes < need || (need > 0 && !workspace))
    return fail(MX_ERR_INVALID_ARG, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  if (K % 32 != 0) return fail(MX_ERR_UNSUPPORTED_SHAPE, "K %lld is not a multiple of 32", (long long)K);
  if (K >= K_LIMIT)
    return fail(MX_ERR_UNSUPPORTED_SHAPE, "K %lld too large for 32-bit tile offsets", (long long)K);
  if (((T + 255) / 256 + G) * ((N + 255) / 256) >= ((int64_t)1 << 31))
    return fail(MX_ERR_UNSUPPORTED_SHAPE, "grouped GEMM of %lld x %lld needs 2^31 tiles or more",
                (long long)T, (long long)N);
  if (T == 0 || N == 0) return MX_OK;
  if (!offsets || !c) return fail(MX_ERR_INVALID_ARG, "offsets or c is NULL");
  if (K > 0 && (!a || !sa || !b || !sb)) return fail(MX_ERR_INVALID_ARG, "an operand is NULL");
  int dev;
  mx_status st = current_device(&dev);
  if (st != MX_OK) return st;
  hipError_t e;
  if (K == 0) {
    e = mx::launch_fill_zero(c, 2 * T * N, stream);
  } else {
    int cus;
    {
      std::lock_guard<std::mutex> lk(g_mu);
      cus = g_num_cus[dev];
    }
    e = mx::launch_grouped_gemm((int)a_elem, (int)b_elem, G, offsets, T, N, K, a, sa, b, sb, c, cus,
                                stream);
  }
  if (e != hipSuccess) return hip_fail(e, "grouped GEMM kernel launch");
  return MX_OK;
}

mx_status mx_grouped_gemm(int64_t G, const int64_t* offsets, int64_t T, int64_t N, int64_t K,
                          const void* a, const void* sa, const void* b, const void* sb, void* c,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return mx_grouped_gemm_elem(MX_ELEM_E4M3, MX_ELEM_E4M3, G, offsets, T, N, K, a, sa, b, sb, c,
                              workspace, workspace_bytes, stream);
}

mx_status mx_quant_batched_elem(mx_quant_mode mode, mx_elem_type elem, const void* x,
                                int64_t batch, int64_t rows, int64_t cols, void* q, void* s,
                                void* q_t, void* s_t, hipStream_t stream) {
  g_err[0] = '\0';
  if (mode < MX_QUANT_ROW_1x32 || mode > MX_QUANT_BLOCK_32x32)
    return fail(MX_ERR_INVALID_ARG, "unknown quantisation mode %d", (int)mode);
  if (elem != MX_ELEM_E4M3 && elem != MX_ELEM_E5M2)
    return fail(MX_ERR_INVALID_ARG, "unknown element type %d", (int)elem);
  if (batch < 0 || batch > 65535) return fail(MX_ERR_INVALID_ARG, "batch %lld not in [0, 65535]", (long long)batch);
  if (rows < 0 || cols < 0) return fail(MX_ERR_INVALID_ARG, "negative shape [%lld, %lld]",
                                        (long long)rows, (long long)cols);
  if (mul_overflows(rows, cols) || mul_overflows(batch, rows * cols) ||
      batch * rows * cols > (INT64_MAX / 4))
    return fail(MX_ERR_INVALID_ARG, "shape too large");
  const bool need_row = mode == MX_QUANT_ROW_1x32 || mode == MX_QUANT_DUAL_AXIS ||
                        mode == MX_QUANT_BLOCK_32x32;
  const bool need_col = mode == MX_QUANT_COL_1x32 || mode == MX_QUANT_DUAL_AXIS;
  if (cols % 32 != 0)
    return fail(MX_ERR_UNSUPPORTED_SHAPE, "cols %lld is not a multiple of 32", (long long)cols);
  if (mode != MX_QUANT_ROW_1x32 && rows % 32 != 0)
    return fail(MX_ERR_UNSUPPORTED_SHAPE, "rows %lld is not a multiple of 32", (long long)rows);
  if (mode != MX_QUANT_ROW_1x32 && (cols + 127) / 128 > 65535)
    return fail(MX_ERR_UNSUPPORTED_SHAPE, "cols %lld exceeds the column-tile grid", (long long)cols);
  if (batch == 0 || rows == 0 || cols == 0) return MX_OK;
  // 32x32 tiles run the stack as one [batch * rows, cols] matrix (no
  // overflow: batch * rows * cols was checked above and cols > 0)
  if (mode != MX_QUANT_ROW_1x32 &&
      row_tiles_too_large(mode == MX_QUANT_BLOCK_32x32 ? batch * rows : rows))
    return fail(MX_ERR_UNSUPPORTED_SHAPE, "rows %lld exceed the row-tile grid", (long long)rows);
  if (!x) return fail(MX_ERR_INVALID_ARG, "x is NULL");
  if (need_row && (!q || !s)) return fail(MX_ERR_INVALID_ARG, "q and s are required for this mode");
  if (need_col && (!q_t || !s_t))
    return fail(MX_ERR_INVALID_ARG, "q_t and s_t are required for this mode");
  int dev;
  mx_status st = current_device(&dev);
  if (st != MX_OK) return st;
  hipError_t e;
  const int el = (int)elem;
  // row blocks and 32x32 tiles never cross a matrix boundary: the stack is
  // one [batch * rows, cols] matrix for them
  switch (mode) {
    case MX_QUANT_ROW_1x32: e = mx::launch_quant_row(x, batch * rows * cols, q, s, el, stream); break;
    case MX_QUANT_BLOCK_32x32:
      e = mx::launch_quant_tile(3, x, batch * rows, cols, q, s, q_t, s_t, 1, el, stream);
      break;
    case MX_QUANT_COL_1x32: e = mx::launch_quant_tile(1, x, rows, cols, q, s, q_t, s_t, batch, el, stream); break;
    default: e = mx::launch_quant_tile(2, x, rows, cols, q, s, q_t, s_t, batch, el, stream); break;
  }
  if (e != hipSuccess) return hip_fail(e, "quantisation kernel launch");
  return MX_OK;
}

mx_status mx_quant_batched(mx_quant_mode mode, const void* x, int64_t batch, int64_t rows,
                           int64_t cols, void* q, void* s, void* q_t, void* s_t,
                           hipStream_t stream) {
  return mx_quant_batched_elem(mode, MX_ELEM_E4M3, x, batch, rows, cols, q, s, q_t, s_t, stream);
}

int64_t mx_grouped_col_capacity(int64_t T, int64_t G) {
  if (T < 0 || G < 1 || G > (INT64_MAX / 128) - T / 128) return -1;
  return 128 * (T / 128 + G);
}

mx_status mx_quant_grouped_col_elem(mx_elem_type elem, const void* x, int64_t T, int64_t C,
                                    int64_t G, const int64_t* offsets, void* q_t, void* s_t,
                                    hipStream_t stream) {
  g_err[0] = '\0';
  if (elem != MX_ELEM_E4M3 && elem != MX_ELEM_E5M2)
    return fail(MX_ERR_INVALID_ARG, "unknown element type %d", (int)elem);
  if (G < 1 || G > 512) return fail(MX_ERR_INVALID_ARG, "group count %lld not in [1, 512]", (long long)G);
  if (T < 0 || C < 0) return fail(MX_ERR_INVALID_ARG, "negative shape [%lld, %lld]", (long long)T,
                                  (long long)C);
  if (C % 32 != 0) return fail(MX_ERR_UNSUPPORTED_SHAPE, "cols %lld is not a multiple of 32", (long long)C);
  if ((C + 127) / 128 > 65535)
    return fail(MX_ERR_UNSUPPORTED_SHAPE, "cols %lld exceeds the column-tile grid", (long long)C);
  const int64_t cap = mx_grouped_col_capacity(T, G);
  if (cap < 0 || cap >= K_LIMIT)
    return fail(MX_ERR_UNSUPPORTED_SHAPE, "token capacity %lld too large", (long long)cap);
  if (mul_overflows(T, C) || mul_overflows(cap, C)) return fail(MX_ERR_INVALID_ARG, "shape too large");
  if (C == 0) return MX_OK;
  if (!offsets || !q_t || !s_t) return fail(MX_ERR_INVALID_ARG, "offsets, q_t or s_t is NULL");
  if (T > 0 && !x) return fail(MX_ERR_INVALID_ARG, "x is NULL");
  int dev;
  mx_status st = current_device(&dev);
  if (st != MX_OK) return st;
  hipError_t e = mx::launch_quant_grouped_col(x, T, C, G, offsets, cap, q_t, s_t, (int)elem, stream);
  if (e != hipSuccess) return hip_fail(e, "grouped column quantisation kernel launch");
  return MX_OK;
}

mx_status mx_quant_grouped_col(const void* x, int64_t T, int64_t C, int64_t G,
                               const int64_t* offsets, void* q_t, void* s_t, hipStream_t stream) {
  return mx_quant_grouped_col_elem(MX_ELEM_E4M3, x, T, C, G, offsets, q_t, s_t, stream);
}

mx_status mx_grouped_gemm_wgrad_elem(mx_elem_type a_elem, mx_elem_type b_elem, int64_t G,
                                     const int64_t* offsets, int64_t T, int64_t M, int64_t N,
                                     const void* a, const void* sa, const void* b, const void* sb,
                                     void* c, hipStream_t stream) {
  g_err[0] = '\0';
  if ((a_elem != MX_ELEM_E4M3 && a_elem != MX_ELEM_E5M2) ||
      (b_elem != MX_ELEM_E4M3 && b_elem != MX_ELEM_E5M2))
    return fail(MX_ERR_INVALID_ARG, "unknown element type (a %d, b %d)", (int)a_elem, (int)b_elem);
  if (G < 1 || G > 512) return fail(MX_ERR_INVALID_ARG, "group count %lld not in [1, 512]", (long long)G);
  if (T < 0 || M < 0 || N < 0) return fail(MX_ERR_INVALID_ARG, "negative grouped wgrad shape");
  const int64_t cap = mx_grouped_col_capacity(T, G);
  if (cap < 0 || cap >= K_LIMIT)
    return fail(MX_ERR_UNSUPPORTED_SHAPE, "token capacity %lld too large", (long long)cap);
  if (mul_overflows(M, cap) || mul_overflows(N, cap) || mul_overflows(M, N) || mul_overflows(G, M * N))
    return fail(MX_ERR_INVALID_ARG, "grouped wgrad shape too large");
  if (grid_too_large(G * gemm_tiles(M, N)))
    return fail(MX_ERR_UNSUPPORTED_SHAPE, "%lld experts x %lld x %lld output tiles exceed one launch grid",
                (long long)G, (long long)M, (long long)N);
  if (M == 0 || N == 0) return MX_OK;
  if (!offsets || !c || !a || !sa || !b || !sb) return fail(MX_ERR_INVALID_ARG, "a pointer is NULL");
  int dev;
  mx_status st = current_device(&dev);
  if (st != MX_OK) return st;
  int cus;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    cus = g_num_cus[dev];
  }
  hipError_t e = mx::launch_grouped_wgrad((int)a_elem, (int)b_elem, G, offsets, T, M, N, cap, a, sa,
                                          b, sb, c, cus, stream);
  if (e != hipSuccess) return hip_fail(e, "grouped wgrad kernel launch");
  return MX_OK;
}

mx_status mx_grouped_gemm_wgrad(int64_t G, const int64_t* offsets, int64_t T, int64_t M, int64_t N,
                                const void* a, const void* sa, const void* b, const void* sb,
                                void* c, hipStream_t stream) {
  return mx_grouped_gemm_wgrad_elem(MX_ELEM_E4M3, MX_ELEM_E4M3, G, offsets, T, M, N, a, sa, b, sb,
                                    c, stream);
}

}  // extern "C"
