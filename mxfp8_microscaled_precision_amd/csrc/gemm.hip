// MXFP8 GEMMs for gfx950: C[m][n] = sum_k A[m][k] * B[n][k] with E4M3
// operands, one E8M0 scale per 32 K-elements of each operand row, FP32
// accumulation and a BF16 result (torchtitan-npu MXFP8/HiF8 tutorial, "MXFP8
// / HiF8 architecture overview": the forward runs as an FP8 matmul whose
// output is restored to BF16; MoE experts run as a grouped matmul).  The
// grouped form multiplies rows offsets[g] .. offsets[g+1]-1 of the token
// matrix by expert g's weight (MindSpeed RFC "add MXFP8-32x32 quantisation
// support to FSDP", section 2.2: gate_up_proj / down_proj of MoE experts).
// The 32x32 weight variant takes one scale per 32x32 weight tile, and its
// backward-data product reads the one shared FP8 weight transposed (RFC
// sections 3.1 and 3.3.3).  The MFMA lane layout and the shared helpers are
// in gemm_common.h.
//
// Workgroup tile 256 (M) x 256 (N), K step 128 bytes, four waves of 128x128
// (16 accumulators of 32x32 each).  Both operands are staged through a
// double-buffered LDS tile whose 16-byte chunks are XOR-swizzled by row, so
// the fragment reads are free of bank conflicts.
#include "gemm_common.h"

namespace mx {

// One workgroup tile.  Pipeline (two LDS stages, one barrier per K step):
//   phase A of step kt: MFMAs of K half 0 on registers F0, LDS reads of
//     half 1 into F1 interleaved;
//   barrier: every wave has read stage kt, and the loads of stage kt+1 and
//     the scales of step kt+1 have landed (vmcnt(0));
//   phase B: buffer->LDS loads of stage kt+2 into the buffer just released,
//     scale loads of step kt+2, MFMAs of half 1 on F1, LDS reads of half 0 of
//     stage kt+1 into F0 interleaved.
// The loop body has no branches so the scheduler can interleave freely.
//
// Scales.  With LDS_SCALES (K a multiple of the K step and at least four
// steps) the per-row scale bytes of four K steps are staged through LDS like
// the operands: one 16-byte load per row every four steps (rows cost one
// cache line per four steps instead of one per step), read back per step
// with ds_read_u16 at the lane half's two blocks.  When the step count is not
// a multiple of four, the last group's 16 bytes are loaded ending at the
// row's last scale byte (never past it) and read at a matching offset, and
// the group's steps past the end (zero payload from out-of-range loads) get
// scale words 0 (finite).  Otherwise every step loads scale words from
// global memory.
// FAST: 0 = the general variant (any K a multiple of 32); 1 = the pipeline
// with LDS-staged scales, K a multiple of 512; 2 = the same with a partial last
// group of four K steps (K a multiple of 128, at least 512).
// TAIL: with FAST == 2, run only the real steps of the last group (the
// persistent grouped kernel keeps the whole group, which needs fewer
// registers there).
// PFBT: with the transposed weight, prefetch B's K-step slices into L2 too
// (one more register; the one-tile-per-workgroup kernel only).
template <int BMODE, int FAST, int FA = 0, int FB = 0, int OUT = 0, bool TAIL = true,
          bool PFBT = false>
struct Tile {
  static constexpr bool LDS_SCALES = FAST != 0;
  static constexpr bool PARTIAL = FAST == 2;
  const uint8_t* __restrict__ a;
  const uint8_t* __restrict__ sa;
  const uint8_t* __restrict__ b;
  const uint8_t* __restrict__ sb;
  uint16_t* __restrict__ c;
  uint8_t* __restrict__ q_out;  // OUT != 0: row-quantised result (payload, scales)
  uint8_t* __restrict__ s_out;
  int64_t m0, m_end, n0, N, K, nkb;
  int64_t nks;      // K steps
  int64_t last_g;   // LDS_SCALES: index of the last 4-step group
  uint32_t sdelta;  // LDS_SCALES: bytes the last group's load is shifted back by
  lds_u8* st0;  // the two LDS stages (distinct arrays, so the compiler can
  lds_u8* st1;  // tell the loads into one from the reads of the other)
  lds_u8* ss0;  // two scale tiles (LDS_SCALES): [256 rows][16 B] of A, then
  lds_u8* ss1;  // the same of B, covering four K steps

  u32x4 ra, rb, rsa, rsb;
  uint32_t svoff;               // scale-tile load offset of this lane's row
  uint32_t svoff_b, sb_row;     // the same for B's scales; bytes per block index
  // L2 prefetch (the LDS_SCALES pipeline): the first workgroup of each
  // concurrently running group to need a K slice fetches it PF_DIST steps
  // ahead of use; pf_a / pf_b are 0 for the operands this workgroup
  // prefetches and OOB (no memory access) otherwise.
  lds_u8* pf_scratch;           // 2 KB
  uint32_t pf_row, pf_a, pf_b;
  uint32_t pf_row_b;  // PFBT: this lane's line of a K step's slice of B
  uint32_t voff_a, voff_b;      // per-lane offset of this lane's first chunk
  uint32_t a_step, b_step;      // offset between this wave's consecutive chunks
  int64_t srow_a[4], srow_b[4]; // scale row bases

  __device__ __forceinline__ void setup(int wave, int lane) {
    const int64_t mrows = m_end - m0;
    nks = (K + BK - 1) / BK;
    last_g = (nks - 1) >> 2;
    sdelta = (uint32_t)(16 * (last_g + 1) - 4 * nks);  // 16 - 4 * (steps in the last group)
    ra = make_rsrc(a + m0 * K, mrows * K);
    // A: instruction t = wave + 4u covers LDS rows 8t .. 8t+7 (1 KB); lane i
    // lands in row r = 8t + i/8 at physical chunk i%8, holding logical chunk
    // (i%8) ^ swz(r); swz(r) = (4 wave + i/16) & 7 does not depend on u.
    const int sw = (4 * wave + (lane >> 4)) & 7;
    voff_a = (uint32_t)((8 * wave + (lane >> 3)) * K + 16 * ((lane & 7) ^ sw));
    a_step = (uint32_t)(32 * K);
    if (BMODE == GEMM_B_TILE_T) {
      // B stored [K][N]; tile columns n0 .. n0+255.  Instruction t covers LDS
      // rows (k) 4t .. 4t+3 of 256 bytes; lane i -> row 4t + i/16, physical
      // chunk i%16 holding logical chunk (i%16) ^ 2(row & 7).
      // Columns past N feed only outputs that are never stored, and the
      // buffer ends with the weight, so they need no mask.
      // (K >= 1 here: the host writes zeros for K == 0 without a launch)
      const int64_t bbytes = (K - 1) * N + (N - n0);
      rb = make_rsrc(b + n0, bbytes > 0 ? bbytes : 0);
      const int krow = 4 * wave + (lane >> 4);
      const int lc = (lane & 15) ^ (2 * (krow & 7));
      voff_b = (uint32_t)(krow * N + 16 * lc);
      b_step = (uint32_t)(16 * N);
    } else {
      const int64_t nrows = (N - n0) < BN ? (N - n0) : BN;
      rb = make_rsrc(b + n0 * K, nrows * K);
      voff_b = (uint32_t)((8 * wave + (lane >> 3)) * K + 16 * ((lane & 7) ^ sw));
      b_step = (uint32_t)(32 * K);
    }
    const int i = lane & 31;
    const int wm = wave & 1, wn = wave >> 1;
    const int64_t lda = K >> 5;
    if (LDS_SCALES) {
      // scale tiles: wave w loads rows 64w .. 64w+63, one 16-byte chunk
      // (four K steps) per lane; rows past the edge read as zero
      rsa = make_rsrc(sa + m0 * lda, mrows * lda);
      svoff = (uint32_t)((64 * wave + lane) * lda);
      if (BMODE == GEMM_B_ROW) {
        const int64_t nrows = (N - n0) < BN ? (N - n0) : BN;
        rsb = make_rsrc(sb + n0 * lda, nrows * lda);
        svoff_b = svoff;
        sb_row = 1;
      } else if (BMODE == GEMM_B_TILE) {
        // the tile's 8 rows of tile scales, 16 bytes (four K steps) each,
        // loaded by lanes 0..7 of wave 0
        const int64_t tr0 = n0 >> 5, ntr = ((N - n0) >> 5) < 8 ? ((N - n0) >> 5) : 8;
        rsb = make_rsrc(sb + tr0 * lda, ntr * lda);
        svoff_b = lane < 8 ? (uint32_t)(lane * lda) : OOB;
        sb_row = 1;
      } else {
        // transposed weight: tile-scale rows kb (along K) hold the tile
        // columns of N; a 4-step group needs 16 rows x the tile's 8 columns
        // (two dwords), loaded by lanes 0..31 of wave 0.  Columns past N
        // feed only outputs that are never stored.
        const int64_t c0t = n0 >> 5, ldt = N >> 5;
        rsb = make_rsrc(sb + c0t, (nkb - 1) * ldt + (ldt - c0t));
        svoff_b = lane < 32 ? (uint32_t)((lane >> 1) * ldt + 4 * (lane & 1)) : OOB;
        sb_row = (uint32_t)ldt;
      }
    }
    pf_row = (uint32_t)((64 * wave + lane) * K);
    if constexpr (PFBT) {
      // transposed weight [K][N]: a K step's slice of B is 128 rows of 256
      // bytes, two lines per row; lane l of wave w takes row (64 w + l) / 2,
      // line l % 2 (N is a multiple of 128, so both lines lie in the row)
      pf_row_b = (uint32_t)(((64 * wave + lane) >> 1) * N + 128 * (lane & 1));
    }
#pragma unroll
    for (int f = 0; f < 4; f++) {
      int64_t m = m0 + 128 * wm + 32 * f + i;
      m = m < m_end ? m : m_end - 1;
      srow_a[f] = m * lda;
      int64_t n = n0 + 128 * wn + 32 * f + i;
      n = n < N ? n : N - 1;
      srow_b[f] = BMODE == GEMM_B_ROW ? n * lda : (BMODE == GEMM_B_TILE ? (n >> 5) * lda : (n >> 5));
    }
    if (BMODE == GEMM_B_TILE_T && FAST) {
      // four consecutive tile columns from an aligned dword; a wave whose
      // columns lie past N (its results are never stored) reads the last four
      const int64_t c0 = (n0 + 128 * wn) >> 5, last = (N >> 5) - 4;
      srow_b[0] = c0 < last ? c0 : last;
    }
  }

  // buffer -> LDS loads of the K step starting at byte k0 into stage st:
  // chunk u of A and of B for this wave (u = 0 .. CHUNKS-1).  Chunks at or
  // past K read as zero (K is a multiple of 32, so whole 16-byte chunks are
  // in or out).  With FAST (K a multiple of the K step) no real step is
  // partial, and a step past the end gets the base offset OOB: its loads
  // touch no memory.  step_base() is uniform, one scalar select per step.
  __device__ __forceinline__ uint32_t step_base_a(int64_t k0) const {
    return k0 < K ? (uint32_t)k0 : OOB;
  }
  __device__ __forceinline__ uint32_t step_base_b(int64_t k0) const {
    if (BMODE == GEMM_B_TILE_T) return k0 < K ? (uint32_t)k0 * (uint32_t)N : OOB;
    return k0 < K ? (uint32_t)k0 : OOB;
  }

  __device__ __forceinline__ void dma_a(lds_u8* st, int64_t k0, uint32_t base, int u, int wave,
                                        int lane) {
    const int t = wave + 4 * u;
    uint32_t off = voff_a + base + u * a_step;
    if (!FAST) {
      const int lc = (lane & 7) ^ ((4 * wave + (lane >> 4)) & 7);
      off = (k0 + 16 * lc < K) ? off : OOB;
    }
    dma16(st + t * 1024, off, ra);
  }

  __device__ __forceinline__ void dma_b(lds_u8* st, int64_t k0, uint32_t base, int u, int wave,
                                        int lane) {
    const int t = wave + 4 * u;
    uint32_t off = voff_b + base + u * b_step;
    // transposed B: rows at or past K lie beyond the end of its buffer
    if (!FAST && BMODE != GEMM_B_TILE_T) {
      const int lc = (lane & 7) ^ ((4 * wave + (lane >> 4)) & 7);
      off = (k0 + 16 * lc < K) ? off : OOB;
    }
    dma16(st + A_TILE + t * 1024, off, rb);
  }

  __device__ __forceinline__ void issue_stage(lds_u8* st, int64_t k0, int wave, int lane) {
    const uint32_t ba = step_base_a(k0), bb = step_base_b(k0);
#pragma unroll
    for (int u = 0; u < CHUNKS; u++) dma_a(st, k0, ba, u, wave, lane);
#pragma unroll
    for (int u = 0; u < CHUNKS; u++) dma_b(st, k0, bb, u, wave, lane);
  }

  // Scale words of K step kb0 (blocks kb0 .. kb0+3).  load_scales fetches raw
  // words (for the transposed 32x32 weight: four rows of the tile-scale
  // array, one dword = the tiles of four consecutive fragments), and
  // finish_scales turns them into one word per fragment, shifted so that
  // byte s feeds MFMA half s for this lane's half of the wave.  FAST: K is a
  // multiple of the K step (and, transposed, N a multiple of 128), so every
  // word is one aligned dword; steps past the end load a dummy that is never
  // used.
  __device__ __forceinline__ uint32_t scale_word(const uint8_t* base, int64_t kb0) {
    if (FAST) return *(const uint32_t*)(base + (kb0 < nkb ? kb0 : nkb - 4));
    uint32_t r = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) r |= (uint32_t)(kb0 + i < nkb ? base[kb0 + i] : 0x7F) << (8 * i);
    return r;
  }

  __device__ __forceinline__ void load_scales_b(int64_t kb0, uint32_t* rb_) {
    if (BMODE == GEMM_B_TILE_T) {
      const int64_t ld = N >> 5;
      if (FAST) {
        // row kb of the tile scales, tiles of fragments 0..3 (4 bytes)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int64_t kb = kb0 + i < nkb ? kb0 + i : nkb - 1;
          rb_[i] = *(const uint32_t*)(sb + kb * ld + srow_b[0]);
        }
      } else {
#pragma unroll
        for (int f = 0; f < 4; f++) {
          uint32_t v = 0;
#pragma unroll
          for (int i = 0; i < 4; i++)
            v |= (uint32_t)(kb0 + i < nkb ? sb[(kb0 + i) * ld + srow_b[f]] : 0x7F) << (8 * i);
          rb_[f] = v;
        }
      }
    } else {
#pragma unroll
      for (int f = 0; f < 4; f++) rb_[f] = scale_word(sb + srow_b[f], kb0);
    }
  }

  __device__ __forceinline__ void load_scales(int64_t kb0, uint32_t* ra_, uint32_t* rb_) {
#pragma unroll
    for (int f = 0; f < 4; f++) ra_[f] = scale_word(sa + srow_a[f], kb0);
    load_scales_b(kb0, rb_);
  }

  __device__ __forceinline__ void finish_scales_b(int lane, const uint32_t* rb_, uint32_t* sbr) {
    const int sh = 16 * (lane >> 5);
    if (BMODE == GEMM_B_TILE_T && FAST) {
      // 4x4 byte transpose: word f collects byte f of rows 0..3
      const uint32_t lo01 = __builtin_amdgcn_perm(rb_[1], rb_[0], 0x05010400u);  // r0b0 r1b0 r0b1 r1b1
      const uint32_t hi01 = __builtin_amdgcn_perm(rb_[1], rb_[0], 0x07030602u);  // r0b2 r1b2 r0b3 r1b3
      const uint32_t lo23 = __builtin_amdgcn_perm(rb_[3], rb_[2], 0x05010400u);
      const uint32_t hi23 = __builtin_amdgcn_perm(rb_[3], rb_[2], 0x07030602u);
      uint32_t w[4];
      w[0] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
      w[1] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
      w[2] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
      w[3] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
#pragma unroll
      for (int f = 0; f < 4; f++) sbr[f] = w[f] >> sh;
    } else {
#pragma unroll
      for (int f = 0; f < 4; f++) sbr[f] = rb_[f] >> sh;
    }
  }

  __device__ __forceinline__ void finish_scales(int lane, const uint32_t* ra_, const uint32_t* rb_,
                                                uint32_t* sar, uint32_t* sbr) {
    const int sh = 16 * (lane >> 5);
#pragma unroll
    for (int f = 0; f < 4; f++) sar[f] = ra_[f] >> sh;
    finish_scales_b(lane, rb_, sbr);
  }

  // LDS_SCALES: scale-tile loads of the 4-step group whose first block is
  // kb0, and the per-step reads (two blocks per lane: 2g and 2g+1 of step q).
  // The scale tile holds A's rows at [0, 4 KB) and B's scales at [4 KB, ...):
  // per-row words like A's for B_ROW, [8 tile rows][16 B] for B_TILE,
  // [16 block rows][8 B] for B_TILE_T.  The tile-scale loads are issued by
  // wave 0 only (one destination for the whole workgroup); the barrier
  // after wave 0's own vmcnt wait publishes them.
  __device__ __forceinline__ void dma_scales(lds_u8* buf, int64_t kb0, int wave) {
    const bool live = kb0 < nkb;  // none past the end
    // per-row 16-byte loads of the last group end at the row's last byte
    const int64_t kbl = (!PARTIAL || kb0 + 16 <= nkb) ? kb0 : nkb - 16;
    dma16(buf + wave * 1024, live ? svoff + (uint32_t)kbl : OOB, rsa);
    uint32_t offb = live ? svoff_b + (uint32_t)(BMODE == GEMM_B_TILE_T ? kb0 : kbl) * sb_row : OOB;
    if (BMODE == GEMM_B_TILE_T && PARTIAL) {
      // lane 2r + h loads row kb0 + r of the tile scales; rows past the end
      // read zero
      const int lane = threadIdx.x & 63;
      offb = kb0 + (lane >> 1) < nkb ? offb : OOB;
    }
    if (BMODE == GEMM_B_ROW)
      dma16(buf + 4096 + wave * 1024, offb, rsb);
    else if (BMODE == GEMM_B_TILE) {
      if (wave == 0) dma16(buf + 4096, offb, rsb);
    } else {
      if (wave == 0) dma4(buf + 4096, offb, rsb);
    }
  }

  // Scale words of step kst, step q = kst % 4 of its group (q is passed as a
  // compile-time value where the caller has it).
  __device__ __forceinline__ void read_scales(const lds_u8* buf, int q, int64_t kst, int wm, int wn,
                                              int lane, uint32_t* sar, uint32_t* sbr) {
    const int g = lane >> 5, i = lane & 31;
    const uint32_t dl = (PARTIAL && (kst >> 2) == last_g) ? sdelta : 0u;  // the last group's shift
    const uint32_t keep = (!PARTIAL || kst < nks) ? 0xFFFFFFFFu : 0u;   // steps past the end: 0
#pragma unroll
    for (int f = 0; f < 4; f++)
      sar[f] = keep & *(const lds_u16*)(buf + (128 * wm + 32 * f + i) * 16 + 4 * q + dl + 2 * g);
    if (BMODE == GEMM_B_ROW) {
#pragma unroll
      for (int f = 0; f < 4; f++)
        sbr[f] = keep & *(const lds_u16*)(buf + 4096 + (128 * wn + 32 * f + i) * 16 + 4 * q + dl + 2 * g);
    } else {
      // one word per fragment (B_TILE: the tile row's four blocks of step q)
      // or per block (B_TILE_T: the wave's four tile columns of block 4q+i),
      // the same for every lane; finish_scales_b shapes them per lane
      uint32_t w[4];
#pragma unroll
      for (int f = 0; f < 4; f++)
        w[f] = keep & (BMODE == GEMM_B_TILE
                   ? *(const __attribute__((address_space(3))) uint32_t*)(buf + 4096 + (4 * wn + f) * 16 + 4 * q + dl)
                   : *(const __attribute__((address_space(3))) uint32_t*)(buf + 4096 + (4 * q + f) * 8 + 4 * wn));
      finish_scales_b(lane, w, sbr);
    }
  }

  template <int S>
  __device__ __forceinline__ void read_frags(const lds_u8* st, int wm, int wn, int lane, v8i* af,
                                             v8i* bf) {
    const int g = lane >> 5, i = lane & 31;
#pragma unroll
    for (int f = 0; f < 4; f++) af[f] = read_frag(st, 128 * wm + 32 * f + i, S, g);
#pragma unroll
    for (int f = 0; f < 4; f++) {
      if (BMODE == GEMM_B_TILE_T)
        bf[f] = read_frag_t(st + A_TILE, 128 * wn + 32 * f, S, lane);
      else
        bf[f] = read_frag(st + A_TILE, 128 * wn + 32 * f + i, S, g);
    }
  }

  template <int S>
  __device__ __forceinline__ void mma(const v8i* af, const v8i* bf, const uint32_t* sar,
                                      const uint32_t* sbr, v16f (&acc)[4][4]) {
    mma_tile<S, FA, FB>(af, bf, sar, sbr, acc);
  }

  // LDS fragment reads and vector-memory loads issued per K half
  static constexpr int DS_READS = BMODE == GEMM_B_TILE_T ? 8 + 16 : 16;
  static constexpr int SCALE_LOADS = (BMODE == GEMM_B_TILE_T && !FAST) ? 4 + 16 : 8;

  template <int NDS, int NVM>
  __device__ __forceinline__ static void interleave() {
    interleave_ops<NDS, NVM>();
  }

  // One K step on stage `cur`, prefetching into `nxt` (see the pipeline
  // description above).
  __device__ __forceinline__ void step(lds_u8* cur, lds_u8* nxt, int64_t kt, int wave, int wm,
                                       int wn, int lane, uint32_t* sc_a, uint32_t* sc_b,
                                       uint32_t* nx_a, uint32_t* nx_b, v8i* f0a, v8i* f0b,
                                       v8i* f1a, v8i* f1b, v16f (&acc)[4][4]) {
    // phase A: raw scales of step kt+1 land by the barrier
    load_scales((kt + 1) * (BK / 32), nx_a, nx_b);
    read_frags<1>(cur, wm, wn, lane, f1a, f1b);
    mma<0>(f0a, f0b, sc_a, sc_b, acc);
    interleave<DS_READS, SCALE_LOADS>();
    wait_vm_all();  // this wave's loads of stage kt+1 have landed ...
    __syncthreads();  // ... and every wave's; every wave is done reading `cur`
    // keep the scale arithmetic below the barrier (it would otherwise be
    // scheduled next to its load and wait on it)
#pragma unroll
    for (int f = 0; f < 4; f++) asm volatile("" : "+v"(nx_a[f]), "+v"(nx_b[f]));
    // phase B: fragment reads of stage kt+1 and loads of stage kt+2 into `cur`
    const int64_t k2 = (kt + 2) * BK;
    const uint32_t ba = step_base_a(k2), bb = step_base_b(k2);
    const int g = lane >> 5, i = lane & 31;
#pragma unroll
    for (int f = 0; f < 4; f++) {
      f0a[f] = read_frag(nxt, 128 * wm + 32 * f + i, 0, g);
      dma_a(cur, k2, ba, 2 * f, wave, lane);
      dma_a(cur, k2, ba, 2 * f + 1, wave, lane);
    }
#pragma unroll
    for (int f = 0; f < 4; f++) {
      if (BMODE == GEMM_B_TILE_T)
        f0b[f] = read_frag_t(nxt + A_TILE, 128 * wn + 32 * f, 0, lane);
      else
        f0b[f] = read_frag(nxt + A_TILE, 128 * wn + 32 * f + i, 0, g);
      dma_b(cur, k2, bb, 2 * f, wave, lane);
      dma_b(cur, k2, bb, 2 * f + 1, wave, lane);
    }
    mma<1>(f1a, f1b, sc_a, sc_b, acc);
    interleave<DS_READS, 0>();
    finish_scales(lane, nx_a, nx_b, sc_a, sc_b);
  }

  // One K step with LDS-staged scales; U = kt % 4.  `sread` holds the scale
  // tile of step kt+1; at U == 0 the tile of the next group is loaded into
  // `sdma` (its previous contents were last read two barriers earlier).
  // Every mode waits with vmcnt(2): the two most recent vector-memory ops of
  // every step are its L2 prefetches, which nothing waits for.
  template <int U>
  __device__ __forceinline__ void step_ls(lds_u8* cur, lds_u8* nxt, const lds_u8* sread,
                                          lds_u8* sdma, int64_t kt, int wave, int wm, int wn,
                                          int lane, uint32_t* sc_a, uint32_t* sc_b,
                                          uint32_t* nx_a, uint32_t* nx_b, v8i* f0a, v8i* f0b,
                                          v8i* f1a, v8i* f1b, v16f (&acc)[4][4]) {
    // phase A
    read_frags<1>(cur, wm, wn, lane, f1a, f1b);
    mma<0>(f0a, f0b, sc_a, sc_b, acc);
    interleave<DS_READS, 0>();
    wait_vm_but_prefetch();
    __syncthreads();
    // phase B
    if (U == 0) dma_scales(sdma, (kt + 4) * (BK / 32), wave);
    read_scales(sread, (U + 1) & 3, kt + 1, wm, wn, lane, nx_a, nx_b);
    const int64_t k2 = (kt + 2) * BK;
    const uint32_t ba = step_base_a(k2), bb = step_base_b(k2);
    const int g = lane >> 5, i = lane & 31;
#pragma unroll
    for (int f = 0; f < 4; f++) {
      f0a[f] = read_frag(nxt, 128 * wm + 32 * f + i, 0, g);
      dma_a(cur, k2, ba, 2 * f, wave, lane);
      dma_a(cur, k2, ba, 2 * f + 1, wave, lane);
    }
#pragma unroll
    for (int f = 0; f < 4; f++) {
      if (BMODE == GEMM_B_TILE_T)
        f0b[f] = read_frag_t(nxt + A_TILE, 128 * wn + 32 * f, 0, lane);
      else
        f0b[f] = read_frag(nxt + A_TILE, 128 * wn + 32 * f + i, 0, g);
      dma_b(cur, k2, bb, 2 * f, wave, lane);
      dma_b(cur, k2, bb, 2 * f + 1, wave, lane);
    }
    prefetch(kt + PF_DIST, wave);
    mma<1>(f1a, f1b, sc_a, sc_b, acc);
    interleave<DS_READS + 8, 0>();
#pragma unroll
    for (int f = 0; f < 4; f++) {
      sc_a[f] = nx_a[f];
      sc_b[f] = nx_b[f];
    }
  }

  // L2 prefetch of K step kt (pf_a / pf_b select the workgroups that issue
  // it; steps past the end touch no memory)
  __device__ __forceinline__ void prefetch(int64_t kt, int wave) {
    const int64_t kp = kt * BK;
    const uint32_t live = kp < K ? 0u : OOB;
    prefetch_lines(pf_scratch + wave * 512, (pf_row + (uint32_t)kp) | pf_a | live, ra);
    uint32_t ob = pf_row + (uint32_t)kp;
    if constexpr (PFBT) ob = pf_row_b + (uint32_t)kp * (uint32_t)N;
    prefetch_lines(pf_scratch + wave * 512 + 256, ob | pf_b | live, rb);
  }

  // The K loop of the LDS_SCALES pipeline after its prologue: step 0's scale
  // words in sc_a / sc_b and its half-0 fragments in f0a / f0b.
  __device__ __forceinline__ void kloop_ls(v16f (&acc)[4][4], int wave, int lane, uint32_t* sc_a,
                                           uint32_t* sc_b, v8i* f0a, v8i* f0b) {
    const int wm = wave & 1, wn = wave >> 1;
    const int64_t nk = (K + BK - 1) / BK;
    uint32_t nx_a[4], nx_b[4];
    v8i f1a[4], f1b[4];
    // with PARTIAL && TAIL the last group runs only its real steps (the
    // loads the skipped ones would issue lie past the end)
    const int64_t kend = (PARTIAL && TAIL) ? 4 * last_g : nk;
    for (int64_t j = 0; 4 * j < kend; j++) {
      const int64_t kt = 4 * j;
      lds_u8* scur = (j & 1) ? ss1 : ss0;
      lds_u8* snxt = (j & 1) ? ss0 : ss1;
      step_ls<0>(st0, st1, scur, snxt, kt, wave, wm, wn, lane, sc_a, sc_b, nx_a, nx_b, f0a, f0b,
                 f1a, f1b, acc);
      step_ls<1>(st1, st0, scur, snxt, kt + 1, wave, wm, wn, lane, sc_a, sc_b, nx_a, nx_b, f0a,
                 f0b, f1a, f1b, acc);
      step_ls<2>(st0, st1, scur, snxt, kt + 2, wave, wm, wn, lane, sc_a, sc_b, nx_a, nx_b, f0a,
                 f0b, f1a, f1b, acc);
      step_ls<3>(st1, st0, snxt, snxt, kt + 3, wave, wm, wn, lane, sc_a, sc_b, nx_a, nx_b, f0a,
                 f0b, f1a, f1b, acc);
    }
    if (PARTIAL && TAIL) {
      const int64_t j = last_g, kt = 4 * j, r = nk - kt;  // 1 .. 3 real steps
      lds_u8* scur = (j & 1) ? ss1 : ss0;
      lds_u8* snxt = (j & 1) ? ss0 : ss1;
      step_ls<0>(st0, st1, scur, snxt, kt, wave, wm, wn, lane, sc_a, sc_b, nx_a, nx_b, f0a, f0b,
                 f1a, f1b, acc);
      if (r > 1)
        step_ls<1>(st1, st0, scur, snxt, kt + 1, wave, wm, wn, lane, sc_a, sc_b, nx_a, nx_b, f0a,
                   f0b, f1a, f1b, acc);
      if (r > 2)
        step_ls<2>(st0, st1, scur, snxt, kt + 2, wave, wm, wn, lane, sc_a, sc_b, nx_a, nx_b, f0a,
                   f0b, f1a, f1b, acc);
    }
  }

  // The LDS_SCALES prologue in two parts, for a persistent caller that
  // issues the next tile's first loads before it stores the current result:
  // issue_first() loads stage 0 and the first scale group (17 or 18 ops
  // per wave), issue_second() stage 1 (16 ops); run_issued() waits for
  // stage 0 only (all but the ops issued after it: stage 1's, and with
  // `stored` the NST result stores of the halves epilogue issued between
  // the two: 32 for BF16, 33 quantised) and runs the K loop into acc.
  __device__ __forceinline__ void issue_first(int wave, int lane) {
    issue_stage(st0, 0, wave, lane);
    dma_scales(ss0, 0, wave);
  }
  __device__ __forceinline__ void issue_second(int wave, int lane) { issue_stage(st1, BK, wave, lane); }
  template <int NST = 32>
  __device__ __forceinline__ void run_issued(v16f (&acc)[4][4], int wave, int lane, bool stored) {
    static_assert(LDS_SCALES, "the split prologue is the LDS-staged-scale pipeline's");
    const int wm = wave & 1, wn = wave >> 1;
#pragma unroll
    for (int x = 0; x < 4; x++)
#pragma unroll
      for (int y = 0; y < 4; y++) acc[x][y] = (v16f){};
    if (stored)
      wait_vm<NST + 2 * CHUNKS>();
    else
      wait_vm<2 * CHUNKS>();
    __syncthreads();
    uint32_t sc_a[4], sc_b[4];
    v8i f0a[4], f0b[4];
    read_scales(ss0, 0, 0, wm, wn, lane, sc_a, sc_b);
    // the steps' vmcnt(2) waits assume the latest two ops are prefetches
    prefetch(2, wave);
    read_frags<0>(st0, wm, wn, lane, f0a, f0b);
    kloop_ls(acc, wave, lane, sc_a, sc_b, f0a, f0b);
  }

  __device__ __forceinline__ void run() {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    setup(wave, lane);
    v16f acc[4][4];
#pragma unroll
    for (int x = 0; x < 4; x++)
#pragma unroll
      for (int y = 0; y < 4; y++) acc[x][y] = (v16f){};
    const int64_t nk = (K + BK - 1) / BK;
    uint32_t sc_a[4], sc_b[4], nx_a[4], nx_b[4];
    v8i f0a[4], f0b[4], f1a[4], f1b[4];

    if (LDS_SCALES) {
      // nk >= 4; the last group may be partial
      issue_stage(st0, 0, wave, lane);
      dma_scales(ss0, 0, wave);
      wait_vm_all();
      __syncthreads();
      read_scales(ss0, 0, 0, wm, wn, lane, sc_a, sc_b);
      issue_stage(st1, BK, wave, lane);
      // The steps wait with vmcnt(2), which leaves the two most recent loads
      // in flight: those must be prefetches, never stage loads.  So the
      // prologue ends with the two prefetches of stage 2.
      prefetch(2, wave);
      read_frags<0>(st0, wm, wn, lane, f0a, f0b);
      kloop_ls(acc, wave, lane, sc_a, sc_b, f0a, f0b);
    } else {
      issue_stage(st0, 0, wave, lane);
      load_scales(0, nx_a, nx_b);
      wait_vm_all();
      finish_scales(lane, nx_a, nx_b, sc_a, sc_b);
      __syncthreads();
      issue_stage(st1, BK, wave, lane);
      read_frags<0>(st0, wm, wn, lane, f0a, f0b);
      int64_t kt = 0;
      for (; kt + 1 < nk; kt += 2) {
        step(st0, st1, kt, wave, wm, wn, lane, sc_a, sc_b, nx_a, nx_b, f0a, f0b, f1a, f1b, acc);
        step(st1, st0, kt + 1, wave, wm, wn, lane, sc_a, sc_b, nx_a, nx_b, f0a, f0b, f1a, f1b, acc);
      }
      if (kt < nk)
        step(st0, st1, kt, wave, wm, wn, lane, sc_a, sc_b, nx_a, nx_b, f0a, f0b, f1a, f1b, acc);
    }
    // no load may still be writing this workgroup's LDS when it ends (or
    // when the stage buffers take the result)
    wait_vm_all();
    if (OUT == 0) {
      __syncthreads();  // every wave is past its last read of the stages
      store_tile_bf16_lds(acc, st0, st1, c, N, m0, m_end, n0, N, wm, wn, wave, lane);
    } else {
      store_tile_q<OUT - 1>(acc, q_out, s_out, N, m0, m_end, n0, N, wm, wn, lane);
    }
  }
};


// OUT: 0 = BF16 result in c; 1 / 2 = the result quantised in 1x32 blocks
// along N with E4M3 / E5M2 payload into q, s (fused producer).
template <int BMODE, int FAST, int FA, int FB, int OUT>
__global__ void __launch_bounds__(NT)
gemm_kernel(const uint8_t* __restrict__ a, const uint8_t* __restrict__ sa,
            const uint8_t* __restrict__ b, const uint8_t* __restrict__ sb, uint16_t* __restrict__ c,
            uint8_t* __restrict__ q, uint8_t* __restrict__ s, int64_t M, int64_t N, int64_t K) {
  __shared__ __attribute__((aligned(16))) uint8_t smem0[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t smem1[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sscale[2 * SCALE_TILE];
  __shared__ __attribute__((aligned(16))) uint8_t spf[2048];
  const int64_t nm = (M + BM - 1) / BM, nn = (N + BN - 1) / BN;
  int64_t mt, nt;
  tile_of(blockIdx.x, nm, nn, mt, nt);
  constexpr bool PFBT = BMODE == GEMM_B_TILE_T && FAST == 1;
  Tile<BMODE, FAST, FA, FB, OUT, true, PFBT> t;
  t.a = a;
  t.sa = sa;
  t.b = b;
  t.sb = sb;
  t.c = c;
  t.q_out = q;
  t.s_out = s;
  t.m0 = mt * BM;
  t.m_end = (mt + 1) * BM < M ? (mt + 1) * BM : M;
  t.n0 = nt * BN;
  t.N = N;
  t.K = K;
  t.nkb = K >> 5;
  t.st0 = (lds_u8*)smem0;
  t.st1 = (lds_u8*)smem1;
  t.ss0 = (lds_u8*)sscale;
  t.ss1 = (lds_u8*)sscale + SCALE_TILE;
  // tile_of runs GM m-tiles x (32 / GM) n-tiles per XCD at a time: A slices
  // are first needed by n-tiles at multiples of 32 / GM, B slices by m-tiles
  // at multiples of GM
  t.pf_scratch = (lds_u8*)spf;
  t.pf_a = (nt % (32 / GM_TILES) == 0) ? 0u : OOB;
  // the transposed weight [K][N] prefetches its own slices (PFBT), and
  // only where each XCD walks its own eighth of the order: measured 3-4.6%
  // faster there (32768 x 18432 x 7168), 0.6-0.9% slower with the runs
  // dealt in turn
  if (BMODE == GEMM_B_TILE_T)
    t.pf_b = (PFBT && mt % GM_TILES == 0 && !tile_runs_rr((uint32_t)nm, (uint32_t)nn)) ? 0u : OOB;
  else
    t.pf_b = (mt % GM_TILES == 0) ? 0u : OOB;
  t.run();
}

// Persistent form of the GEMM (K a multiple of 512, BF16 result with N a
// multiple of 8, or with OUT the fused producer's quantised result with N a
// multiple of 256): one workgroup per compute unit walks tiles bid, bid +
// grid, ... of gemm_kernel's tile map (a grid that is a multiple of 8 keeps
// every tile on the XCD it has there, index mod 8, so an XCD still runs the
// same 32-tile groups at a time), and each tile's stage 0 loads while the
// previous tile's result is stored.
template <int BMODE, int FA, int FB, int OUT = 0>
__global__ void __launch_bounds__(NT)
gemm_persistent_kernel(const uint8_t* __restrict__ a, const uint8_t* __restrict__ sa,
                       const uint8_t* __restrict__ b, const uint8_t* __restrict__ sb,
                       uint16_t* __restrict__ c, uint8_t* __restrict__ q, uint8_t* __restrict__ s,
                       int64_t M, int64_t N, int64_t K) {
  __shared__ __attribute__((aligned(16))) uint8_t smem0[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t smem1[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sscale[2 * SCALE_TILE];
  __shared__ __attribute__((aligned(16))) uint8_t spf[2048];
  __shared__ __attribute__((aligned(16))) uint8_t ssq[OUT ? 2048 : 16];  // OUT: a tile's scales
  const int64_t nm = (M + BM - 1) / BM, nn = (N + BN - 1) / BN, tiles = nm * nn;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  typedef Tile<BMODE, 1, FA, FB, 0> T1;
  auto make = [&](int64_t t, T1& tl) {
    int64_t mt, nt;
    tile_of(t, nm, nn, mt, nt);
    tl.a = a;
    tl.sa = sa;
    tl.b = b;
    tl.sb = sb;
    tl.c = c;
    tl.q_out = nullptr;
    tl.s_out = nullptr;
    tl.m0 = mt * BM;
    tl.m_end = (mt + 1) * BM < M ? (mt + 1) * BM : M;
    tl.n0 = nt * BN;
    tl.N = N;
    tl.K = K;
    tl.nkb = K >> 5;
    tl.st0 = (lds_u8*)smem0;
    tl.st1 = (lds_u8*)smem1;
    tl.ss0 = (lds_u8*)sscale;
    tl.ss1 = (lds_u8*)sscale + SCALE_TILE;
    tl.pf_scratch = (lds_u8*)spf;
    tl.pf_a = (nt % (32 / GM_TILES) == 0) ? 0u : OOB;
    // B only where each XCD walks its own eighth of the order: where the
    // XCDs take the runs of one group in turn, prefetching B measured
    // 2.5-4.6% slower on the K = 18432 and 32768 shapes (N = 7168)
    tl.pf_b = (mt % GM_TILES == 0 && BMODE != GEMM_B_TILE_T &&
               !tile_runs_rr((uint32_t)nm, (uint32_t)nn)) ? 0u : OOB;
  };
  int64_t t = blockIdx.x;
  if (t >= tiles) return;
  T1 tl;
  make(t, tl);
  tl.setup(wave, lane);
  tl.issue_first(wave, lane);
  bool stored = false;
  for (;;) {
    tl.issue_second(wave, lane);
    v16f acc[4][4];
    tl.template run_issued<OUT ? 33 : 32>(acc, wave, lane, stored);
    const int64_t m0 = tl.m0, m_end = tl.m_end, n0 = tl.n0;
    // every load has landed (none may still be writing LDS) and every wave
    // is past its last read of the stage and scale buffers
    wait_vm_all();
    __syncthreads();
    t += gridDim.x;
    const bool more = __builtin_amdgcn_readfirstlane((int)(t < tiles)) != 0;
    // 32x32 weights: the lane index through an empty asm, so that what the
    // next tile's setup and this tile's store derive from it is computed
    // here, not hoisted out of the loop and held in registers across the K
    // loop (it was, and they spilled); the 1x32 form fits without it and
    // measured 1-2% faster on the long-K shapes that way
    int ln = lane;
    if constexpr (BMODE != GEMM_B_ROW) asm volatile("" : "+v"(ln));
    if (more) {
      make(t, tl);
      tl.setup(wave, ln);
      tl.issue_first(wave, ln);
    }
    if constexpr (OUT == 0)
      store_tile_bf16_lds_halves(acc, (lds_u8*)smem1, c, N, m0, m_end, n0, N, wave & 1, wave >> 1,
                                 wave, ln);
    else
      store_tile_q_lds_halves<OUT - 1>(acc, (lds_u8*)smem1, (lds_u8*)ssq, q, s, N, m0, m_end, n0,
                                       wave & 1, wave >> 1, wave, ln);
    stored = true;
    if (!more) break;
  }
}

// Persistent grouped GEMM: every workgroup derives the tile list from the
// device-side offsets (clamped into [0, T] and made non-decreasing, so bad
// offsets can never address outside the operands) and walks it with a static
// stride.  Tile t -> (group g, m tile within g, n tile).
// FA / FB: element formats of the token rows and of the expert weights.
template <int FAST, int FA = 0, int FB = 0, bool OVERLAP = false>
__global__ void __launch_bounds__(NT)
grouped_gemm_kernel(int64_t G, const int64_t* __restrict__ offsets, int64_t T, int64_t N,
                    int64_t K, const uint8_t* __restrict__ a, const uint8_t* __restrict__ sa,
                    const uint8_t* __restrict__ b, const uint8_t* __restrict__ sb,
                    uint16_t* __restrict__ c) {
  __shared__ __attribute__((aligned(16))) uint8_t smem0[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t smem1[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sscale[2 * SCALE_TILE];
  __shared__ __attribute__((aligned(16))) uint8_t spf[2048];
  __shared__ int64_t s_off[MAX_GROUPS + 1];
  __shared__ int64_t s_pre[MAX_GROUPS + 1];
  const int64_t nn = (N + BN - 1) / BN;
  for (int64_t g = threadIdx.x; g <= G; g += NT) {
    int64_t o = offsets[g];
    s_off[g] = o < 0 ? 0 : (o > T ? T : o);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t prev = 0, acc = 0;
    for (int64_t g = 0; g < G; g++) {
      int64_t lo = s_off[g] > prev ? s_off[g] : prev;
      int64_t hi = s_off[g + 1] > lo ? s_off[g + 1] : lo;
      s_off[g] = lo;
      prev = lo;
      s_pre[g] = acc;
      acc += ((hi - lo + BM - 1) / BM) * nn;
    }
    s_off[G] = s_off[G] > prev ? s_off[G] : prev;
    s_pre[G] = acc;
  }
  __syncthreads();
  const int64_t total = s_pre[G];
  // contiguous tile runs per XCD
  const int64_t nwg = gridDim.x, bid = blockIdx.x;
  const int64_t wg = (bid & 7) * (nwg >> 3) + (bid >> 3);
  // tile indices fit in 32 bits (the host checks the tile count), so the
  // per-tile arithmetic below is 32-bit
  const uint32_t span = GM_TILES * (uint32_t)nn;
  int64_t g = 0;  // largest g with s_pre[g] <= t: searched once, then advanced
  {
    int64_t hi = G;
    while (hi - g > 1) {
      const int64_t mid = (g + hi) >> 1;
      if (s_pre[mid] <= wg) g = mid; else hi = mid;
    }
  }
  // tile t (t >= wg, non-decreasing along the walk) into tl
  auto make_tile = [&](int64_t t, Tile<GEMM_B_ROW, FAST, FA, FB, 0, false>& tl) {
    while (s_pre[g + 1] <= t) g++;  // s_pre[G] = total > t stops it
    // inside group g, the same grouped order as the dense kernel: runs of
    // GM_TILES m-tiles, n-tiles outer, so 32 consecutive tiles cover
    // GM_TILES m-tiles x (32 / GM_TILES) n-tiles
    const uint32_t local = (uint32_t)(t - s_pre[g]);
    const uint32_t nmg = (uint32_t)((s_off[g + 1] - s_off[g] + BM - 1) / BM);
    const uint32_t run = local / span;
    const uint32_t first = run * GM_TILES;
    const uint32_t gsz = (nmg - first) < (uint32_t)GM_TILES ? (nmg - first) : (uint32_t)GM_TILES;
    const uint32_t in = local - run * span;
    const uint32_t nt = in / gsz;
    const int64_t mt = first + (in - nt * gsz);
    tl.a = a;
    tl.sa = sa;
    tl.b = b + g * N * K;
    tl.sb = sb + g * N * (K >> 5);
    tl.c = c;
    tl.m0 = s_off[g] + mt * BM;
    tl.m_end = (tl.m0 + BM) < s_off[g + 1] ? tl.m0 + BM : s_off[g + 1];
    tl.n0 = (int64_t)nt * BN;
    tl.N = N;
    tl.K = K;
    tl.nkb = K >> 5;
    tl.st0 = (lds_u8*)smem0;
    tl.st1 = (lds_u8*)smem1;
    tl.ss0 = (lds_u8*)sscale;
    tl.ss1 = (lds_u8*)sscale + SCALE_TILE;
    // as in the dense kernel: A slices are first needed by n-tiles at
    // multiples of 32 / GM_TILES, B slices by the first m-tile of a run
    // (B only with more than 32 n-tiles, as in the persistent dense GEMM)
    tl.pf_scratch = (lds_u8*)spf;
    tl.pf_a = (nt % (32 / GM_TILES) == 0) ? 0u : OOB;
    tl.pf_b = (mt == first && nn > 32) ? 0u : OOB;
  };
  if constexpr (OVERLAP) {
    // The next tile's stage 0 goes to stage buffer 0 while the result
    // leaves through buffer 1 (32 stores per wave); its stage 1 follows, and
    // it waits for stage 0 only, so the stores drain under its first K step.
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int64_t t = wg;
    if (t >= total) return;
    Tile<GEMM_B_ROW, FAST, FA, FB, 0, false> tl;
    make_tile(t, tl);
    tl.setup(wave, lane);
    tl.issue_first(wave, lane);
    bool stored = false;
    for (;;) {
      tl.issue_second(wave, lane);
      v16f acc[4][4];
      tl.run_issued(acc, wave, lane, stored);
      const int64_t m0 = tl.m0, m_end = tl.m_end, n0 = tl.n0;
      // every load has landed (none may still be writing LDS) and every wave
      // is past its last read of the stage and scale buffers
      wait_vm_all();
      __syncthreads();
      t += nwg;
      // uniform, and said so: a branch the compiler took for divergent would
      // carry the next tile's descriptors out of it in vector registers
      const bool more = __builtin_amdgcn_readfirstlane((int)(t < total)) != 0;
      if (more) {
        make_tile(t, tl);
        tl.setup(wave, lane);
        tl.issue_first(wave, lane);
      }
      store_tile_bf16_lds_halves(acc, (lds_u8*)smem1, c, N, m0, m_end, n0, N, wave & 1, wave >> 1,
                                 wave, lane);
      stored = true;
      if (!more) break;
    }
    return;
  }
  for (int64_t t = wg; t < total; t += nwg) {
    Tile<GEMM_B_ROW, FAST, FA, FB, 0, false> tl;
    make_tile(t, tl);
    tl.run();
  }
}

// Zero fill of `nbytes` bytes at p (any alignment): the bytes before the
// first 16-byte boundary and after the last are written one by one by the
// first workgroup, the 16-byte-aligned middle with 16-byte stores.
__global__ void fill_zero_kernel(uint8_t* __restrict__ p, int64_t head, int64_t n16,
                                 int64_t nbytes) {
  uint4* mid = (uint4*)(p + head);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * blockDim.x)
    mid[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0) {
    for (int64_t i = threadIdx.x; i < head; i += blockDim.x) p[i] = 0;
    for (int64_t i = head + 16 * n16 + threadIdx.x; i < nbytes; i += blockDim.x) p[i] = 0;
  }
}

template <int BMODE, int FAST>
static void launch_gemm_fmt(int a_elem, int b_elem, dim3 grid, const uint8_t* A, const uint8_t* SA,
                            const uint8_t* B, const uint8_t* SB, uint16_t* C, int64_t M, int64_t N,
                            int64_t K, hipStream_t stream) {
#define MX_GEMM_LAUNCH(FA_, FB_)                                                                  \
  hipLaunchKernelGGL((gemm_kernel<BMODE, FAST, FA_, FB_, 0>), grid, dim3(NT), 0, stream, A, SA, B,  \
                     SB, C, (uint8_t*)nullptr, (uint8_t*)nullptr, M, N, K)
  if (a_elem == 0 && b_elem == 0) MX_GEMM_LAUNCH(0, 0);
  else if (a_elem == 1 && b_elem == 0) MX_GEMM_LAUNCH(1, 0);
  else if (a_elem == 0 && b_elem == 1) MX_GEMM_LAUNCH(0, 1);
  else MX_GEMM_LAUNCH(1, 1);
#undef MX_GEMM_LAUNCH
}

// Pipeline variant for a shape (the FAST parameter of Tile): 1 when K is a
// multiple of 512, 2 when it is a multiple of 128 and at least 512, else 0;
// the transposed 32x32 weight also needs N % 128 == 0 for the pipeline.
static int pipe_of(int bmode, int64_t N, int64_t K) {
  if (K % BK != 0 || K < 4 * BK || (bmode == GEMM_B_TILE_T && N % 128 != 0)) return 0;
  return K % (4 * BK) == 0 ? 1 : 2;
}

hipError_t launch_gemm(int bmode, int a_elem, int b_elem, int64_t M, int64_t N, int64_t K,
                       const void* a, const void* sa, const void* b, const void* sb, void* c,
                       int num_cus, hipStream_t stream) {
  if ((a_elem != 0 && a_elem != 1) || (b_elem != 0 && b_elem != 1)) return hipErrorInvalidValue;
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  dim3 grid((unsigned)tiles);
  const uint8_t *A = (const uint8_t*)a, *SA = (const uint8_t*)sa, *B = (const uint8_t*)b,
                *SB = (const uint8_t*)sb;
  uint16_t* C = (uint16_t*)c;
  const int pipe = pipe_of(bmode, N, K);
  // with more tiles than compute units the GEMM runs persistent, one
  // tile's stores overlapping the next tile's first loads (the halves
  // epilogue: whole 8-column chunks, 32-bit store offsets).  With a 32x32
  // weight only for K up to 4096: there the overlap gains 3-4% (K = 2048),
  // while the transposed weight at K = 7168-18432 measured 9% slower
  // persistent than one tile per workgroup
  const int64_t cus = (num_cus > 0 ? num_cus : 256) / 8 * 8;
  if (pipe == 1 && N % 8 == 0 && (int64_t)BM * N * 2 < ((int64_t)1 << 31) && cus >= 8 &&
      tiles > cus && (bmode == GEMM_B_ROW || K <= 4096)) {
    dim3 pg((unsigned)cus);
#define MX_GEMMP_LAUNCH(BM_, FA_, FB_)                                                            \
  hipLaunchKernelGGL((gemm_persistent_kernel<BM_, FA_, FB_>), pg, dim3(NT), 0, stream, A, SA, B, SB, \
                     C, (uint8_t*)nullptr, (uint8_t*)nullptr, M, N, K)
#define MX_GEMMP_FMT(BM_)                                            \
  do {                                                               \
    if (a_elem == 0 && b_elem == 0) MX_GEMMP_LAUNCH(BM_, 0, 0);      \
    else if (a_elem == 1 && b_elem == 0) MX_GEMMP_LAUNCH(BM_, 1, 0); \
    else if (a_elem == 0 && b_elem == 1) MX_GEMMP_LAUNCH(BM_, 0, 1); \
    else MX_GEMMP_LAUNCH(BM_, 1, 1);                                 \
  } while (0)
    if (bmode == GEMM_B_ROW) MX_GEMMP_FMT(GEMM_B_ROW);
    else if (bmode == GEMM_B_TILE) MX_GEMMP_FMT(GEMM_B_TILE);
    else MX_GEMMP_FMT(GEMM_B_TILE_T);
#undef MX_GEMMP_FMT
#undef MX_GEMMP_LAUNCH
    return hipGetLastError();
  }
#define MX_GEMM_MODE(BM_)                                                                         \
  do {                                                                                            \
    if (pipe == 1) launch_gemm_fmt<BM_, 1>(a_elem, b_elem, grid, A, SA, B, SB, C, M, N, K, stream); \
    else if (pipe == 2)                                                                           \
      launch_gemm_fmt<BM_, 2>(a_elem, b_elem, grid, A, SA, B, SB, C, M, N, K, stream);            \
    else launch_gemm_fmt<BM_, 0>(a_elem, b_elem, grid, A, SA, B, SB, C, M, N, K, stream);         \
  } while (0)
  switch (bmode) {
    case GEMM_B_ROW:
      MX_GEMM_MODE(GEMM_B_ROW);
      break;
    case GEMM_B_TILE:
      MX_GEMM_MODE(GEMM_B_TILE);
      break;
    case GEMM_B_TILE_T:
      MX_GEMM_MODE(GEMM_B_TILE_T);
      break;
    default:
      return hipErrorInvalidValue;
  }
#undef MX_GEMM_MODE
  return hipGetLastError();
}

hipError_t launch_gemm_q(int bmode, int out_elem, int64_t M, int64_t N, int64_t K, const void* a,
                         const void* sa, const void* b, const void* sb, void* q, void* s,
                         int num_cus, hipStream_t stream) {
  if ((out_elem != 0 && out_elem != 1) || N % 32 != 0) return hipErrorInvalidValue;
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  dim3 grid((unsigned)tiles);
  const uint8_t *A = (const uint8_t*)a, *SA = (const uint8_t*)sa, *B = (const uint8_t*)b,
                *SB = (const uint8_t*)sb;
  uint8_t *Q = (uint8_t*)q, *S = (uint8_t*)s;
  const int pipe = pipe_of(bmode, N, K);
  // persistent as the BF16 GEMM (same rule), its result quantised through
  // the LDS halves epilogue (whole 256-byte payload rows, 8-byte scale
  // pieces: N a multiple of 256); not with the transposed 32x32 weight,
  // whose persistent form would spill there
  const int64_t cus = (num_cus > 0 ? num_cus : 256) / 8 * 8;
  if (pipe == 1 && N % 256 == 0 && (int64_t)BM * N < ((int64_t)1 << 31) && cus >= 8 &&
      tiles > cus && (bmode == GEMM_B_ROW || (bmode == GEMM_B_TILE && K <= 4096))) {
    dim3 pg((unsigned)cus);
#define MX_GEMMPQ_LAUNCH(BM_, OUT_)                                                               \
  hipLaunchKernelGGL((gemm_persistent_kernel<BM_, 0, 0, OUT_>), pg, dim3(NT), 0, stream, A, SA, B, \
                     SB, (uint16_t*)nullptr, Q, S, M, N, K)
#define MX_GEMMPQ_OUT(BM_)                        \
  do {                                            \
    if (out_elem == 0) MX_GEMMPQ_LAUNCH(BM_, 1);  \
    else MX_GEMMPQ_LAUNCH(BM_, 2);                \
  } while (0)
    if (bmode == GEMM_B_ROW) MX_GEMMPQ_OUT(GEMM_B_ROW);
    else MX_GEMMPQ_OUT(GEMM_B_TILE);
#undef MX_GEMMPQ_OUT
#undef MX_GEMMPQ_LAUNCH
    return hipGetLastError();
  }
#define MX_GEMMQ_LAUNCH(BM_, KA_)                                                                 \
  do {                                                                                            \
    if (out_elem == 0)                                                                            \
      hipLaunchKernelGGL((gemm_kernel<BM_, KA_, 0, 0, 1>), grid, dim3(NT), 0, stream, A, SA, B, SB, \
                         (uint16_t*)nullptr, Q, S, M, N, K);                                      \
    else                                                                                          \
      hipLaunchKernelGGL((gemm_kernel<BM_, KA_, 0, 0, 2>), grid, dim3(NT), 0, stream, A, SA, B, SB, \
                         (uint16_t*)nullptr, Q, S, M, N, K);                                      \
  } while (0)
#define MX_GEMMQ_MODE(BM_)                                                                        \
  do {                                                                                            \
    if (pipe == 1) MX_GEMMQ_LAUNCH(BM_, 1);                                                       \
    else if (pipe == 2) MX_GEMMQ_LAUNCH(BM_, 2);                                                  \
    else MX_GEMMQ_LAUNCH(BM_, 0);                                                                 \
  } while (0)
  switch (bmode) {
    case GEMM_B_ROW:
      MX_GEMMQ_MODE(GEMM_B_ROW);
      break;
    case GEMM_B_TILE:
      MX_GEMMQ_MODE(GEMM_B_TILE);
      break;
    case GEMM_B_TILE_T:
      MX_GEMMQ_MODE(GEMM_B_TILE_T);
      break;
    default:
      return hipErrorInvalidValue;
  }
#undef MX_GEMMQ_MODE
#undef MX_GEMMQ_LAUNCH
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(int a_elem, int b_elem, int64_t G, const int64_t* offsets, int64_t T,
                               int64_t N, int64_t K, const void* a, const void* sa, const void* b,
                               const void* sb, void* c, int num_cus, hipStream_t stream) {
  if (G > MAX_GROUPS) return hipErrorInvalidValue;
  if ((a_elem != 0 && a_elem != 1) || (b_elem != 0 && b_elem != 1)) return hipErrorInvalidValue;
  const int64_t nn = (N + BN - 1) / BN;
  const int64_t upper = ((T + BM - 1) / BM + G) * nn;
  if (upper >= ((int64_t)1 << 31)) return hipErrorInvalidValue;  // the host rejects it first
  int64_t wgs = num_cus > 0 ? num_cus : 256;
  wgs = (wgs + 7) / 8 * 8;
  if (upper < wgs) wgs = (upper + 7) / 8 * 8;
  if (wgs < 8) wgs = 8;
  const int pipe = pipe_of(GEMM_B_ROW, N, K);
  // the persistent walk overlaps a tile's result stores with the next tile's
  // first loads when the stores can be counted (whole 8-column chunks,
  // 32-bit store offsets: the halves epilogue)
  const bool overlap = N % 8 == 0 && (int64_t)BM * N * 2 < ((int64_t)1 << 31);
#define MX_GROUPED_LAUNCH(P_, FA_, FB_, OV_)                                                      \
  hipLaunchKernelGGL((grouped_gemm_kernel<P_, FA_, FB_, OV_>), dim3((unsigned)wgs), dim3(NT), 0,  \
                     stream, G, offsets, T, N, K, (const uint8_t*)a, (const uint8_t*)sa,          \
                     (const uint8_t*)b, (const uint8_t*)sb, (uint16_t*)c)
#define MX_GROUPED_FMT(P_, OV_)                                                                   \
  do {                                                                                            \
    if (a_elem == 0 && b_elem == 0) MX_GROUPED_LAUNCH(P_, 0, 0, OV_);                             \
    else if (a_elem == 1 && b_elem == 0) MX_GROUPED_LAUNCH(P_, 1, 0, OV_);                        \
    else if (a_elem == 0 && b_elem == 1) MX_GROUPED_LAUNCH(P_, 0, 1, OV_);                        \
    else MX_GROUPED_LAUNCH(P_, 1, 1, OV_);                                                        \
  } while (0)
  // (the partial-group pipeline keeps the plain walk: overlapped, it needs
  // more registers than it has)
  if (pipe == 1 && overlap) MX_GROUPED_FMT(1, true);
  else if (pipe == 1) MX_GROUPED_FMT(1, false);
  else if (pipe == 2) MX_GROUPED_FMT(2, false);
  else MX_GROUPED_FMT(0, false);
#undef MX_GROUPED_FMT
#undef MX_GROUPED_LAUNCH
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, int64_t nbytes, hipStream_t stream) {
  if (nbytes <= 0) return hipSuccess;
  const uintptr_t a = (uintptr_t)p;
  int64_t head = (int64_t)((16 - (a & 15)) & 15);
  if (head > nbytes) head = nbytes;
  const int64_t n16 = (nbytes - head) / 16;
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (uint8_t*)p,
                     head, n16, nbytes);
  return hipGetLastError();
}

}  // namespace mx
