// Attention kernels: block-sparse attention over the kept patch blocks
// (equation "SparseAttn" of "Block-Sparse Global Attention for Efficient
// Multi-View Geometry Transformers", key design 1, with masked entries
// excluded from the softmax), the dense special-token part with its
// log-sum-exp merge (key design 3 and the framework flowchart), and the dense
// path (equation "Attention") used for comparison.
//
// One tile core serves every mode.  A workgroup of QT/32 waves owns QT query
// rows (32 per wave) and walks a list of KT-key tiles: the kept blocks of its
// CSR row (sparse), every tile (dense), a range of tiles (split-K for the
// special queries) or the special-token tiles (patch queries x special keys).
//
// Data flow per key tile, per wave (32x32x16 MFMAs: bf16 for the scores,
// float16 for P V):
//   S^T (keys x queries) = K Q^T : K rows from LDS are the A operand, the
//     wave's 32 query rows stay in registers as the B operand.  Lane l then
//     holds the 16 scores of query l%32 for one half of each 32-key sub-tile.
//   softmax in float32 (exp2 with log2(e)/8 folded into one FMA).
//   O^T (dims x queries) += V^T P^T : P^T is exactly the accumulator layout
//     converted to float16 (the B operand), V^T comes from LDS (A operand),
//     stored as float16 scaled by a power of two per head (see packing).
//     float16 keeps 11 significant bits of every weight where bfloat16 keeps
//     8, so the rounding of P before the product moves an output row by at
//     most 2^-12 of the weighted |V| instead of 2^-9, and costs the same one
//     v_cvt_pk_f16_f32 per two weights.
// For P^T to be usable as the B operand without any data movement, the eight
// keys a lane contributes to one PV instruction must be contiguous in V^T.
// The accumulator rows of lane half hh are i = 8a + 4hh + c; loading K row
// pi(i) (bits 2 and 3 of i swapped) into A row i makes them the keys
// 16m + 8hh + e, e = 0..7, i.e. contiguous.
//
// Instruction budget.  On gfx950 an exp2 costs about three FMAs of issue
// time, and every score needs one exp2, one FMA and one add, so the softmax
// is kept to that minimum:
//  * lazy running max: a tile is exponentiated against the running max
//    directly (no rescaling of O) unless its exact max lies more than 15 log2
//    units above it (weights stay below 2^15, inside the float16 range); that
//    max is one v_max3 chain over the tile's scores;
//  * the rare block (first tile, partial tile, or such a jump) masks keys
//    past a partial block, takes the exact max and rescales O and l; full
//    tiles never execute any masking instructions;
//  * the first product of each score accumulator starts from the constant 0.
// Per tile a wave computes all scores, then exponentiates and multiplies by V
// one 32-key sub-tile at a time (the exponentials of one sub-tile run beside
// the P V products of the previous one).  LDS holds one K tile and one V^T
// tile: V^T of a tile loads while its scores run, K of the next tile while
// it is exponentiated, two barriers per tile.  That keeps a 128-row
// workgroup at 32 KB of LDS and at most 168 registers per lane, so three
// waves share each SIMD (three workgroups per compute unit).
//
// K and V are first packed (once per layer) into "packed order": patch
// tokens, padding, special tokens, padding (each segment a multiple of 128),
// K as rows [H][ntot_pad][64] (bf16) and V transposed as [H][64][ntot_pad]
// (float16, V * 2^sigma_h with sigma_h chosen from the head's largest |V| so
// that it lies in [2^14, 2^15); the epilogues multiply by 2^-sigma_h).  Tiles
// reach LDS with buffer_load_dwordx4 ... lds (each lane's 16 bytes land at
// base + 16 * lane: no staging registers, no LDS store instructions); the
// bank swizzle is applied on the global side, the lane that fills LDS chunk
// (row, physical chunk pc) fetching logical chunk pc ^ swizzle(row).  Every
// wave fetches its share of both the K and the V^T tile.
#include "bsga_internal.hpp"
#include "tile_common.hpp"

namespace bsga {

// kSparseFused:  patch queries x (kept patch blocks, then every special
//                tile) in one online softmax: the final patch rows; with
//                AttnArgs::patch_only, the kept patch blocks alone (the
//                patch-only result)
// kDense:        every query x every key
// kSpecialSplit: special queries x a range of key tiles (split-K partials)
// kPatchSpecial: patch queries x special tiles, merged by log-sum-exp into
//                the patch rows already in O/LSE
// kSparseTail:   kSparseFused, except that the rows of each XCD's last,
//                partial round of workgroups are split into tail_pieces pieces
//                of consecutive key tiles, listed piece-major after the XCD's
//                whole rows: the in-order dispatch then spreads that round
//                over every slot, and concurrent pieces read the same key range
//                of consecutive rows; tail_merge_kernel combines the pieces.
//                Given a workspace (B <= 4096), each head's query blocks are
//                worked longest kept list first (row_order_kernel), so that
//                the workgroups an XCD runs at once hold rows of similar
//                length and the last round holds the shortest ones
enum Mode { kDense = 1, kSpecialSplit = 2, kPatchSpecial = 3, kSparseFused = 4, kSparseTail = 5 };

// most pieces per row of the last round (kSparseTail)
constexpr int kMaxTailPieces = 16;

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* kp;
  const uint16_t* vt;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  uint16_t* o;
  float* lse;
  float* part_o;   // [H][ns_pad][nsplit][64]
  float* part_ml;  // [H][ns_pad][nsplit][2]
  const int* vsig; // [H] power-of-two exponent of the packed V^T
  Dims d;
  int n_items;
  int q_tiles;
  int nsplit;
  int tiles_per_split;
  int rows_per_xcd;  // kSparseTail: rows of each XCD (as xcd_item)
  int tail_m;        // kSparseTail: workgroup slots per XCD (one round)
  int tail_pieces;   // kSparseTail: pieces per row of the last round
  int patch_only;    // kSparseFused: skip the special tiles
  // b = 64 run as aligned pairs (attn_kernel's PAIR, kSparseFused /
  // kSparseTail at QT = KT = 128): query tile I holds query blocks 2I, 2I + 1, key tile J key blocks
  // 2J, 2J + 1; pair_cols[(h Bp + I) Bp + n] = J | act << 28 lists, in
  // ascending J, the key tiles that hold a block kept by either query block,
  // act bit 2 hq + kh set iff query block 2I + hq keeps key block 2J + kh;
  // pair_len[h Bp + I] entries; Bp = ceil(B / 2)
  const int32_t* pair_cols;
  const int32_t* pair_len;
  // kSparseFused / kSparseTail at b = 128: optional order of each head's
  // query blocks (row_perm[h B + p] = the block worked p-th); null: identity
  const int32_t* row_perm;
  // attn_kernel<..., O32 = true>: [H][N][64] float32 copy of the final rows
  // (the value O holds before its bf16 rounding), for the backward
  float* o32;
};

// A tile is exponentiated against a stale running max as long as its exact
// max is at most 15 log2 units above it: weights then stay below 2^15 (plus
// the FMA's last-bit rounding), inside the float16 range (65504) the P V
// product takes them in, and sums over any sequence length stay far below
// float32 overflow.
constexpr float kLazySlack = 15.f;

// Fourth word of a raw buffer resource (byte addressing, 32-bit data format)
constexpr int kBufWord3 = 0x00020000;

// QT query rows per workgroup (QT / 32 waves), KT keys per tile, WPE waves
// per SIMD targeted (bounds the registers of a wave to 512 / WPE).
// PAIR: b = 64 blocks run as aligned pairs (AttnArgs::pair) on QT = KT = 128
// O32: training mode: P enters the P V product as a float16 pair hi + lo
// (about 22 significant bits, against 11 for hi alone) and the final rows are
// also written as float32 to AttnArgs::o32, so that the backward can take
// D = dO . O from them
template <int QT, int KT, int MODE, int WPE, bool PAIR = false, bool O32 = false>
__global__ __launch_bounds__(2 * QT) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void attn_kernel(
    AttnArgs a) {
  constexpr int NW = QT / 32;       // waves
  constexpr int NS = KT / 32;       // 32-key sub-tiles
  constexpr int VROW = KT / 8;      // 16-byte chunks per V^T row
  constexpr int KCH = 8 * KT;       // chunks of a K tile (= chunks of a V^T tile)
  constexpr int LPW = KCH / (64 * NW);  // 64-chunk loads per wave per K (and V^T) tile
  // patch blocks are one query tile; a kept block spans TPB key tiles
  constexpr int TPB = QT / KT;
  static_assert(LPW >= 2 && LPW % 2 == 0 && (KT == 64 || LPW % 4 == 0), "tile loads");
  static_assert(TPB >= 1 && QT % KT == 0, "tile shape");
  __shared__ u32x4 smem[2 * KCH];   // the K tile, then the V^T tile

  const Dims& d = a.d;
  const int T = lid_x(), lane = T & 63;
  const int w = __builtin_amdgcn_readfirstlane(T >> 6);  // wave index, uniform
  const int l32 = lane & 31, hh = lane >> 5;

  // What the tile loop works on: head h, the query tile starting at packed
  // row qp0, and its list of nt key tiles (a CSR row, then the special tiles;
  // a range of tiles; or every tile).
  int h = 0, qp0 = 0, nt = 0, tile0 = 0, split = 0, nt_csr = 0;
  int piece = -1;         // kSparseTail: the piece of the row, or -1 (whole row)
  size_t piece_slot = 0;  // kSparseTail: its partial's slot
  const int32_t* cols = nullptr;
  {
    int item;
    if constexpr (MODE == kSparseTail) {
      const int x = wg_x() % kXcds, j = wg_x() / kXcds;
      const int r0 = x * a.rows_per_xcd;
      const int n_x = min(a.n_items, r0 + a.rows_per_xcd) - r0;
      if (n_x <= 0) return;
      const int full = n_x / a.tail_m * a.tail_m, rem = n_x - full;
      if (j < full) {
        item = r0 + j;
      } else {
        const int q = j - full;
        if (q >= rem * a.tail_pieces) return;
        const int t = q % rem;
        piece = q / rem;
        item = r0 + full + t;
        // every XCD before the last holds rows_per_xcd rows
        piece_slot = ((size_t)x * (a.rows_per_xcd % a.tail_m) + t) * a.tail_pieces + piece;
      }
    } else {
      item = xcd_item(wg_x(), a.n_items);
      if (item < 0) return;
    }
    if constexpr (MODE == kSparseFused || MODE == kSparseTail) {
      if constexpr (PAIR) {
        const int bp = (d.B + 1) >> 1;
        h = item / bp;
        qp0 = (item - h * bp) * QT;
        cols = a.pair_cols + (size_t)item * bp;
        nt_csr = max(0, min(a.pair_len[item], bp));
      } else {
        h = item / d.B;
        const int row = a.row_perm ? h * d.B + a.row_perm[item] : item;
        qp0 = (row - h * d.B) * QT;
        const int r0 = a.row_ptr[row];
        cols = a.col_idx + r0;
        nt_csr = max(0, min(a.row_ptr[row + 1] - r0, d.B));  // a valid row never exceeds B
      }
      nt = nt_csr * TPB + (a.patch_only ? 0 : d.ns_pad / KT);
    } else if constexpr (MODE == kDense) {
      h = item / a.q_tiles;
      qp0 = (item - h * a.q_tiles) * QT;
      nt = d.ntot_pad / KT;
    } else if constexpr (MODE == kSpecialSplit) {
      const int per_h = a.q_tiles * a.nsplit;
      h = item / per_h;
      const int rem = item - h * per_h;
      const int qt = rem / a.nsplit;
      split = rem - qt * a.nsplit;
      qp0 = d.np_pad + qt * QT;
      tile0 = split * a.tiles_per_split;
      nt = max(0, min(a.tiles_per_split, d.ntot_pad / KT - tile0));
    } else {
      h = item / a.q_tiles;
      qp0 = (item - h * a.q_tiles) * QT;
      tile0 = d.np_pad / KT;
      nt = d.ns_pad / KT;
    }
    // everything above is wave-uniform; keep it in scalar registers
    h = __builtin_amdgcn_readfirstlane(h);
    qp0 = __builtin_amdgcn_readfirstlane(qp0);
    nt = __builtin_amdgcn_readfirstlane(nt);
    nt_csr = __builtin_amdgcn_readfirstlane(nt_csr);
    tile0 = __builtin_amdgcn_readfirstlane(tile0);
  }
  // 2^-sigma_h: undoes the power-of-two scale of the head's packed V^T
  const float unscale = __builtin_amdgcn_ldexpf(1.f, -a.vsig[h]);
  // Position of tile n, in two steps so that the global load of a CSR entry
  // can be issued long before its value is consumed: tile_raw(n) loads the
  // entry (always from an in-bounds slot of the row), tile_kp0(n, raw) turns
  // it into the tile's first packed key.  Kept block j of the row covers tiles
  // j TPB .. j TPB + TPB - 1.
  constexpr bool kCsr = MODE == kSparseFused || MODE == kSparseTail;
  auto tile_raw = [&](int n) -> int {
    if constexpr (kCsr) {
      return nt_csr > 0 ? cols[min(n / TPB, nt_csr - 1)] : 0;
    } else {
      return 0;
    }
  };
  auto tile_kp0 = [&](int n, int raw) -> int {
    raw = __builtin_amdgcn_readfirstlane(raw);
    if constexpr (kCsr) {
      const int nb = nt_csr * TPB;
      if (n >= nb) return d.np_pad + min(n - nb, d.ns_pad / KT - 1) * KT;
      const int last = (PAIR ? (d.B + 1) >> 1 : d.B) - 1;
      return min(max(raw & 0x0fffffff, 0), last) * QT + (n % TPB) * KT;
    } else {
      return (tile0 + n) * KT;
    }
  };
  // Sub-tile activity of this wave in tile n (aligned pairs): bit kh for key
  // block 2J + kh, i.e. sub-tiles 2 kh, 2 kh + 1; all active otherwise
  auto tile_act = [&](int n, int raw) -> int {
    if constexpr (kCsr && PAIR) {
      if (n < nt_csr * TPB) return (__builtin_amdgcn_readfirstlane(raw) >> (28 + 2 * (w >> 1))) & 3;
    }
    return 3;
  };
  auto tile_valid = [&](int kp0) -> int {
    return kp0 < d.np_pad ? min(KT, d.np - kp0) : min(KT, d.ns - (kp0 - d.np_pad));
  };

  // ---- direct-to-LDS tile loads into the K slot and the V^T slot.  Every
  // wave issues LPW loads of 64 x 16 B per K tile and LPW per V^T tile; load
  // i of wave w fills chunks (LPW w + i) * 64 + lane.  The swizzle of the row
  // a lane fills depends on i only through i mod 2 (K, and V^T of 64-key
  // tiles) or i mod 4 (V^T of 128-key tiles), so a few per-lane byte offsets
  // cover all loads.
  const uint32_t vrow_bytes = (uint32_t)d.ntot_pad * 2;
  const char* kbase = nullptr;
  const char* vbase = nullptr;
  uint32_t koff[2], voff[4];
  {
    const int r0 = lane >> 3, pc = lane & 7;
#pragma unroll
    for (int j = 0; j < 2; ++j) koff[j] = (uint32_t)(r0 * 128 + 16 * (pc ^ swz_k(8 * j + r0)));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (KT == 128) {
        const int v0 = lane >> 4, vc = lane & 15;
        voff[j] = (uint32_t)v0 * vrow_bytes + 16 * (vc ^ swz_v<128>(4 * j + v0));
      } else {
        voff[j] = (uint32_t)r0 * vrow_bytes + 16 * (pc ^ swz_v<64>(8 * (j & 1) + r0));
      }
    }
  }
  // Loads go through buffer resources (the head's K rows, the head's V^T
  // rows): the per-lane part of the address is the 32-bit offset above, the
  // tile's position a scalar offset, so no 64-bit per-lane addresses are kept.
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
  __amdgpu_buffer_rsrc_t krs, vrs;
  auto set_head = [&](int hd) {
    kbase = (const char*)a.kp + (size_t)hd * d.ntot_pad * kHeadDim * 2;
    vbase = (const char*)a.vt + (size_t)hd * kHeadDim * vrow_bytes;
    krs = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, 0, d.ntot_pad * kHeadDim * 2, kBufWord3);
    vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, 0, kHeadDim * vrow_bytes, kBufWord3);
  };
  // (the tile position is wave-uniform; readfirstlane keeps it a scalar
  // offset, so each load is one instruction)
  auto issue_k = [&](int kp0) {
    kp0 = __builtin_amdgcn_readfirstlane(kp0);
    lds_u32x4* dst = (lds_u32x4*)&smem[w * LPW * 64];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int blk = LPW * w + i;  // 64-chunk block of the K tile: rows 8 blk .. 8 blk + 7
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (__attribute__((address_space(3))) void*)(dst + i * 64),
                                               16, koff[i & 1], (kp0 + 8 * blk) * 128, 0, 0);
    }
  };
  auto issue_v = [&](int kp0) {
    kp0 = __builtin_amdgcn_readfirstlane(kp0);
    lds_u32x4* dst = (lds_u32x4*)&smem[KCH + w * LPW * 64];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int blk = LPW * w + i;
      const int row0 = KT == 128 ? 4 * blk : 8 * blk;  // first V^T row of the block
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (__attribute__((address_space(3))) void*)(dst + i * 64),
                                               16, voff[i & 3], row0 * vrow_bytes + kp0 * 2, 0, 0);
    }
  };

  // ---- operand reads.  Per-lane LDS byte offsets within a slot: K rows of
  // sub-tile 0 for k-step m (sub-tile t adds t * 32 rows); V^T dims l32 at
  // the keys of (sub-tile t, half h2) (dims 32 + l32 add 32 rows).  Every
  // read is one base register plus an immediate offset.
  uint32_t kadr[4], vadr[NS][2];
  {
    const int R0 = pi_row(l32);
#pragma unroll
    for (int m = 0; m < 4; ++m) kadr[m] = (uint32_t)(R0 * 8 + ((4 * hh + m) ^ swz_k(R0))) * 16;
#pragma unroll
    for (int t = 0; t < NS; ++t)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
        vadr[t][h2] = (uint32_t)(l32 * VROW + ((4 * t + 2 * h2 + hh) ^ swz_v<KT>(l32))) * 16;
  }
  constexpr uint32_t kSlotBytes = KCH * 16, kSubK = 32 * 8 * 16, kVHalf = 32 * VROW * 16;
  auto lds_op = [&](uint32_t off) -> bf16x8 {
    return as_bf16x8(*(const u32x4*)((const char*)smem + off));
  };
  auto lds_op16 = [&](uint32_t off) -> f16x8 {
    return __builtin_bit_cast(f16x8, *(const u32x4*)((const char*)smem + off));
  };

  // ---- softmax state of the wave's 32 query rows.  Lane half hh holds
  // dims [32hh, 32hh + 32) of query row qrow as the B operand, and the
  // running max (log2 units: scores * log2(e)/8) and sum.
  bf16x8 qop[4];
  f32x16 o0, o1;
  float m_run, l_run;
  const int qrow = qp0 + 32 * w + l32;
  // kSpecialSplit: a wave whose 32 rows all lie past the last special token
  // skips its scores and P V products; it still issues its share of every
  // tile load and meets every barrier
  const bool idle = MODE == kSpecialSplit && qp0 - d.np_pad + 32 * w >= d.ns;

  // Rare block: masking of a partial tile, exact max, rescaling.  Score r of
  // sub-tile t is key 32 t + pi(8 (r / 4) + 4 hh + r % 4) = kc + 8 hh with
  // kc = 32 t + 16 (r / 8) + 4 (r / 4 % 2) + r % 4.
  auto rare = [&](f32x16 (&s)[NS], float mx, int valid) {
    if (valid < KT) {
      const int lim = valid - 8 * hh;
      mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < NS; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kc = 32 * t + 16 * (r >> 3) + 4 * ((r >> 2) & 1) + (r & 3);
          if (kc >= lim) s[t][r] = -INFINITY;
          mx = fmaxf(mx, s[t][r]);
        }
    }
    const float m_new = fmaxf(m_run, xor32_max(mx) * kScaleLog2);
    const float alpha = fast_exp2(m_run - m_new);  // 0 on the first tile
    o0 *= alpha;
    o1 *= alpha;
    l_run *= alpha;
    m_run = m_new;
  };
  // partial tile, or its exact max (either lane half) more than kLazySlack
  // log2 units above the running max
  auto needs_rare = [&](float mx, int valid) -> bool {
    return valid < KT || __any(!(mx * kScaleLog2 - m_run <= kLazySlack));
  };

  // Tiles n0 .. n1 - 1 of the current segment, from a fresh softmax state.
  // Per tile the wave computes every score (the maxima folded in as they
  // come), decides the rare block, then exponentiates and multiplies by V^T
  // one 32-key sub-tile at a time (the exponentials of one sub-tile run
  // beside the P V products of the previous one).  CSR entries run two tiles
  // ahead: the entry of tile n+2 is loaded during iteration n and consumed
  // after that iteration's waits.
  auto run_tiles = [&](int n0, int n1) {
    {
      const int qtok = packed_token(qrow, d);
      const u32x4* src =
          (const u32x4*)(a.q + ((size_t)h * d.n + (qtok < 0 ? 0 : qtok)) * kHeadDim) + 4 * hh;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        u32x4 t = u32x4{0, 0, 0, 0};
        if (qtok >= 0) t = src[m];
        qop[m] = as_bf16x8(t);
      }
    }
    o0 = f32x16{};
    o1 = f32x16{};
    m_run = -INFINITY;
    l_run = 0.f;
    set_head(h);
    if (n1 <= n0) return;
    int raw_cur = tile_raw(n0), raw_nxt = tile_raw(n0 + 1);
    issue_k(tile_kp0(n0, raw_cur));
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // (aligned pairs: a wave's first tile with any active sub-tile is its
    // first block)
    bool fresh = true;
    for (int n = n0; n < n1; ++n) {
      // V^T(n) fills its slot (free since the previous closing barrier) while
      // the scores of tile n run
      const int kp_n = tile_kp0(n, raw_cur);
      issue_v(kp_n);
      const int act = idle ? 0 : tile_act(n, raw_cur);
      const int raw_after = tile_raw(n + 2);
      f32x16 s[NS];
      if (act != 0) {
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < NS; ++t) {
          if (act & (1 << (2 * t / NS))) {
#pragma unroll
            for (int m = 0; m < 4; ++m)
              s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_op(kadr[m] + t * kSubK), qop[m],
                                                             m == 0 ? f32x16{} : s[t], 0, 0, 0);
            // a plain chain: the backend folds it into one v_max3 per two scores
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
          } else {
            s[t] = f32x16{} - INFINITY;  // an inactive sub-tile weighs nothing
          }
        }
        const int valid = tile_valid(kp_n);
        if (fresh || needs_rare(mx, valid)) rare(s, mx, valid);
        fresh = false;
      }
      // V^T(n) has landed and every wave is done with K(n): K(n+1) fills the
      // K slot while tile n is exponentiated and multiplied by V^T
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (n + 1 < n1) issue_k(tile_kp0(n + 1, raw_nxt));
      float ls = 0.f;
      // the exponential / P V stretch runs at raised issue priority, so that a
      // wave in it keeps the SIMD's other waves (typically in their score
      // MFMAs) from starving the VALU
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int t = 0; t < NS; ++t) {
        if (!(act & (1 << (2 * t / NS)))) continue;
        // the sub-tile's V^T operands are read first and may not be sunk, so
        // the LDS latency hides behind the exponentials
        f16x8 va[2], vb[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          va[h2] = lds_op16(kSlotBytes + vadr[t][h2]);
          vb[h2] = lds_op16(kSlotBytes + vadr[t][h2] + kVHalf);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          f32x8 e8;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            e8[e] = fast_exp2(fmaf(s[t][8 * h2 + e], kScaleLog2, -m_run));
            ls += e8[e];
          }
          const f16x8 pb = __builtin_convertvector(e8, f16x8);
          o0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[h2], pb, o0, 0, 0, 0);
          o1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(vb[h2], pb, o1, 0, 0, 0);
          if constexpr (O32) {
            f32x8 rem;
#pragma unroll
            for (int e = 0; e < 8; ++e) rem[e] = e8[e] - (float)pb[e];
            const f16x8 pl = __builtin_convertvector(rem, f16x8);
            o0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[h2], pl, o0, 0, 0, 0);
            o1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(vb[h2], pl, o1, 0, 0, 0);
          }
        }
      }
      __builtin_amdgcn_s_setprio(0);
      l_run += ls;
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      raw_cur = raw_nxt;
      raw_nxt = raw_after;
    }
  };

  // ---- epilogues.  o_u[4a + c] holds O^T[32u + 8a + 4hh + c][query row qrow]
  // (times 2^sigma_h).  Unnormalised float32 partial of the wave's 32 rows (V's
  // scale undone), with the running max (log2 units, or raw-score units if
  // `raw`) and the row sum.
  auto store_partial = [&](float* po_base, float* pml, bool raw) {
    const float l_tot = xor32_sum(l_run);
    float4* po = (float4*)po_base;
    const float u = unscale;
#pragma unroll
    for (int aa = 0; aa < 4; ++aa) {
      po[(8 * aa + 4 * hh) / 4] =
          make_float4(o0[4 * aa] * u, o0[4 * aa + 1] * u, o0[4 * aa + 2] * u, o0[4 * aa + 3] * u);
      po[(32 + 8 * aa + 4 * hh) / 4] =
          make_float4(o1[4 * aa] * u, o1[4 * aa + 1] * u, o1[4 * aa + 2] * u, o1[4 * aa + 3] * u);
    }
    if (hh == 0) {
      pml[0] = raw ? m_run / kScaleLog2 : m_run;
      pml[1] = l_tot;
    }
  };
  // final rows of O (bf16) and LSE; kPatchSpecial merges into the rows present
  auto store_rows = [&]() {
    const float l_tot = xor32_sum(l_run);
    const int qtok = packed_token(qrow, d);
    if (qtok < 0) return;
    const float inv = l_tot > 0.f ? unscale / l_tot : 0.f;
    // natural-log LSE: (m_run + log2 l) ln 2
    const float lse = l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    uint16_t* orow = a.o + ((size_t)h * d.n + qtok) * kHeadDim;
    float* lrow = a.lse + (size_t)h * d.n + qtok;
    float cp = 0.f, cs = inv, lse_out = lse;
    if constexpr (MODE == kPatchSpecial) {
      const float lse_p = *lrow;
      const float M = fmaxf(lse_p, lse);
      const float wp = lse_p == -INFINITY ? 0.f : expf(lse_p - M);
      const float ws = lse == -INFINITY ? 0.f : expf(lse - M);
      const float den = wp + ws;
      cp = den > 0.f ? wp / den : 0.f;
      cs = den > 0.f ? ws * inv / den : 0.f;
      lse_out = den > 0.f ? M + logf(den) : -INFINITY;
    }
    auto store_half = [&](const f32x16 ou, int u) {
#pragma unroll
      for (int aa = 0; aa < 4; ++aa) {
        u32x2* dst = (u32x2*)(orow + 32 * u + 8 * aa + 4 * hh);
        f32x4 x;
#pragma unroll
        for (int c = 0; c < 4; ++c) x[c] = ou[4 * aa + c] * cs;
        if constexpr (MODE == kPatchSpecial) {
          const u32x2 old = *dst;
          x[0] += cp * __uint_as_float(old[0] << 16);
          x[1] += cp * __uint_as_float(old[0] & 0xffff0000u);
          x[2] += cp * __uint_as_float(old[1] << 16);
          x[3] += cp * __uint_as_float(old[1] & 0xffff0000u);
        }
        *dst = __builtin_bit_cast(u32x2, __builtin_convertvector(x, bf16x4));
        if constexpr (O32)
          *(f32x4*)(a.o32 + ((size_t)h * d.n + qtok) * kHeadDim + 32 * u + 8 * aa + 4 * hh) = x;
      }
    };
    store_half(o0, 0);
    store_half(o1, 1);
    if (hh == 0) *lrow = lse_out;
  };

  if constexpr (MODE == kSparseTail) {
    if (piece < 0) {
      run_tiles(0, nt);
      store_rows();
    } else {
      run_tiles(nt * piece / a.tail_pieces, nt * (piece + 1) / a.tail_pieces);
      const size_t row = piece_slot * QT + 32 * w + l32;
      store_partial(a.part_o + row * kHeadDim, a.part_ml + row * 2, false);
    }
  } else {
    run_tiles(0, nt);
    if constexpr (MODE == kSpecialSplit) {
      const int sq = qrow - d.np_pad;
      const size_t slot = ((size_t)h * d.ns_pad + sq) * a.nsplit + split;
      // raw-score units for the reduction
      store_partial(a.part_o + slot * kHeadDim, a.part_ml + slot * 2, true);
    } else {
      store_rows();
    }
  }
}

// ---------------------------------------------------------------------------
// Split-K reduction for the special queries: one wave per (head, special
// token), one lane per dimension.  The splits' (max, sum) pairs are read one
// per lane, 64 at a time, and broadcast; the partial rows are then summed in
// split order with their loads independent of the running sums.
__global__ __launch_bounds__(256) void special_reduce_kernel(const float* __restrict__ part_o,
                                                             const float* __restrict__ part_ml,
                                                             uint16_t* __restrict__ o,
                                                             float* __restrict__ lse, Dims d,
                                                             int nsplit, float* __restrict__ o32) {
  const int item = wg_x() * 4 + (lid_x() >> 6);
  const int lane = lid_x() & 63;
  if (item >= d.H * d.ns) return;
  const int h = item / d.ns, s = item - h * d.ns;
  const size_t base = ((size_t)h * d.ns_pad + s) * nsplit;
  float M = -INFINITY;
  for (int c = lane; c < nsplit; c += 64) M = fmaxf(M, part_ml[(base + c) * 2]);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
  float L = 0.f, acc = 0.f;
  for (int c0 = 0; c0 < nsplit; c0 += 64) {
    const int c = c0 + lane, cn = min(64, nsplit - c0);
    float wgt = 0.f, lc = 0.f;
    if (c < nsplit) {
      const float mc = part_ml[(base + c) * 2];
      lc = part_ml[(base + c) * 2 + 1];
      // a split without any valid key carries max -inf and adds nothing
      wgt = mc == -INFINITY ? 0.f : fast_exp2((mc - M) * kScaleLog2);
    }
    const float* po = part_o + (base + c0) * kHeadDim + lane;
    // eight splits per step; past the last split the weight (lane >= cn) is
    // 0 and the load repeats the last split's row, so the sums are unchanged
    for (int j0 = 0; j0 < cn; j0 += 8) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u;
        const float wj = __shfl(wgt, j), lj = __shfl(lc, j);
        const float oj = po[(size_t)min(j, cn - 1) * kHeadDim];
        L += wj * lj;
        acc += wj * oj;
      }
    }
  }
  const int tok = special_token(s, d);
  const float val = acc / L;
  o[((size_t)h * d.n + tok) * kHeadDim + lane] = __builtin_bit_cast(uint16_t, (__bf16)val);
  if (o32 != nullptr) o32[((size_t)h * d.n + tok) * kHeadDim + lane] = val;
  if (lane == 0) lse[(size_t)h * d.n + tok] = M * 0.125f + logf(L);
}

// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// Aligned pairs for b = 64 (see AttnArgs): one wave per pair row (head h,
// query tile I) ORs the kept blocks of query blocks 2I and 2I + 1 into a
// 4-bit activity word per key tile J in LDS, then compacts the nonzero words
// in ascending J with a ballot prefix count.
__global__ __launch_bounds__(256) void pair_csr_kernel(const int32_t* __restrict__ row_ptr,
                                                       const int32_t* __restrict__ col_idx,
                                                       Dims d, int32_t* __restrict__ pair_cols,
                                                       int32_t* __restrict__ pair_len) {
  extern __shared__ uint32_t acts[];  // [4 waves][bp]
  const int bp = (d.B + 1) >> 1;
  const int w = lid_x() >> 6, lane = lid_x() & 63;
  const int item = wg_x() * 4 + w;
  const bool live = item < d.H * bp;  // uniform per wave
  uint32_t* f = acts + w * bp;
  if (live)
    for (int j = lane; j < bp; j += 64) f[j] = 0u;
  __syncthreads();
  if (live) {
    const int h = item / bp, i = item - h * bp;
    for (int hq = 0; hq < 2; ++hq) {
      const int qb = 2 * i + hq;
      if (qb >= d.B) break;
      const int r = h * d.B + qb, a0 = row_ptr[r];
      const int n = max(0, min(row_ptr[r + 1] - a0, d.B));
      for (int e = lane; e < n; e += 64) {
        const int j = col_idx[a0 + e];
        if (j >= 0 && j < d.B) atomicOr(&f[j >> 1], 1u << (2 * hq + (j & 1)));
      }
    }
  }
  __syncthreads();
  if (!live) return;
  int pos = 0;
  for (int j0 = 0; j0 < bp; j0 += 64) {
    const int j = j0 + lane;
    const uint32_t v = j < bp ? f[j] : 0u;
    const uint64_t mask = __ballot(v != 0u);
    if (v != 0u)
      pair_cols[(size_t)item * bp + pos + __popcll(mask & ((1ull << lane) - 1))] =
          (int32_t)((uint32_t)j | (v << 28));
    pos += __popcll(mask);
  }
  if (lane == 0) pair_len[item] = pos;
}

static int pair_rows(const Dims& d) { return (d.B + 1) >> 1; }
// pair_csr_kernel keeps four rows of activity words in LDS (64 KB at most)
constexpr int kMaxPairRows = 4096;
static bool pairable(const Dims& d) { return d.b == 64 && pair_rows(d) <= kMaxPairRows; }
static size_t pair_cols_bytes(const Dims& d) {
  return ((size_t)d.H * pair_rows(d) * pair_rows(d) * sizeof(int32_t) + 255) & ~(size_t)255;
}
static size_t pair_len_bytes(const Dims& d) {
  return ((size_t)d.H * pair_rows(d) * sizeof(int32_t) + 255) & ~(size_t)255;
}
static hipError_t launch_pair_csr(const Dims& d, const int32_t* row_ptr, const int32_t* col_idx,
                                  int32_t* pc, int32_t* pl, hipStream_t st) {
  const int items = d.H * pair_rows(d);
  pair_csr_kernel<<<(items + 3) / 4, 256, 4 * pair_rows(d) * sizeof(uint32_t), st>>>(
      row_ptr, col_idx, d, pc, pl);
  return hipGetLastError();
}

// Order of each head's query blocks for the patch rows: longest kept list
// first, ties by block index.  Each block's key (B - length, block) is
// unique, so its position in the order is its rank, the number of smaller
// keys: workgroup (x, h) holds the B keys of head h in LDS and ranks blocks
// 256 x .. 256 x + 255 against all of them (B <= 4096).
__global__ __launch_bounds__(256) void row_order_kernel(const int32_t* __restrict__ row_ptr,
                                                        Dims d, int32_t* __restrict__ perm) {
  __shared__ uint4 key4[1024];
  uint32_t* key = (uint32_t*)key4;
  const int h = wg_y(), T = lid_x();
  const int nb4 = (d.B + 3) >> 2;
  for (int i = T; i < 4 * nb4; i += 256) {
    uint32_t k = 0xffffffffu;  // padding: above every real key
    if (i < d.B) {
      const int r = h * d.B + i;
      const int len = max(0, min(row_ptr[r + 1] - row_ptr[r], d.B));
      k = ((uint32_t)(d.B - len) << 13) | (uint32_t)i;
    }
    key[i] = k;
  }
  __syncthreads();
  const int i = wg_x() * 256 + T;
  if (i >= d.B) return;
  const uint32_t k = key[i];
  int rank = 0;
  for (int j = 0; j < nb4; ++j) {
    const uint4 q = key4[j];
    rank += (q.x < k) + (q.y < k) + (q.z < k) + (q.w < k);
  }
  perm[h * d.B + rank] = i;
}

// Rows that kSparseTail split into pieces: workgroup (XCD x and tail row
// t < tmax, the largest leftover of any XCD; group g of 4 query rows) merges
// the row's float32 partials by
// log-sum-exp and writes O and LSE of those queries; thread T owns dimension
// T % 64 of query 4 g + T / 64.  Many small workgroups keep the partials'
// reads in flight (the merge is memory-bound).
__global__ __launch_bounds__(256) void tail_merge_kernel(const float* __restrict__ part_o,
                                                         const float* __restrict__ part_ml,
                                                         uint16_t* __restrict__ o,
                                                         float* __restrict__ lse, Dims d,
                                                         int rows, int rows_per_xcd, int m,
                                                         int pieces, int tmax, int rows_per_head,
                                                         const int32_t* __restrict__ row_perm,
                                                         float* __restrict__ o32) {
  constexpr int QT = 128;
  const int x = wg_x() / tmax, t = wg_x() % tmax;
  const int r0 = x * rows_per_xcd;
  const int n_x = min(rows, r0 + rows_per_xcd) - r0;
  if (n_x <= 0) return;
  const int full = n_x / m * m, rem = n_x - full;
  if (t >= rem) return;
  const int item = r0 + full + t;
  const size_t slot0 = ((size_t)x * (rows_per_xcd % m) + t) * pieces;
  const int T = lid_x(), dim = T & 63, qr = 4 * wg_y() + (T >> 6);
  float mi[kMaxTailPieces], li[kMaxTailPieces], oi[kMaxTailPieces];
  float M = -INFINITY;
#pragma unroll
  for (int pc = 0; pc < kMaxTailPieces; ++pc) {
    mi[pc] = -INFINITY;
    if (pc >= pieces) continue;
    const size_t row = (slot0 + pc) * QT + qr;
    mi[pc] = part_ml[row * 2];
    li[pc] = part_ml[row * 2 + 1];
    oi[pc] = part_o[row * kHeadDim + dim];
    M = fmaxf(M, mi[pc]);
  }
  float acc = 0.f, l = 0.f;
#pragma unroll
  for (int pc = 0; pc < kMaxTailPieces; ++pc) {
    if (mi[pc] == -INFINITY) continue;  // an empty piece, or no key at all
    const float wgt = fast_exp2(mi[pc] - M);
    acc += oi[pc] * wgt;
    l += li[pc] * wgt;
  }
  const int h = item / rows_per_head;
  const int blk = row_perm ? row_perm[item] : item - h * rows_per_head;
  const int tok = packed_token(blk * QT + qr, d);
  if (tok < 0) return;
  const float val = l > 0.f ? acc / l : 0.f;
  o[((size_t)h * d.n + tok) * kHeadDim + dim] = __builtin_bit_cast(uint16_t, (__bf16)val);
  if (o32 != nullptr) o32[((size_t)h * d.n + tok) * kHeadDim + dim] = val;
  if (dim == 0)
    lse[(size_t)h * d.n + tok] = l > 0.f ? (M + __log2f(l)) * 0.69314718055994531f : -INFINITY;
}

// ---------------------------------------------------------------------------
// Packing: K rows and transposed V in packed order, 64 keys per workgroup.
//
// V^T is stored as float16 so that the P V product can take P as float16
// (11 significant bits).  Every bf16 value times a power of two is exact in
// float16 inside its normal range, so the head's V is scaled by 2^sigma_h
// with its largest |V| in [2^14, 2^15) (below the float16 maximum 65504);
// values more than 2^28 below that maximum land among the float16 subnormals
// with an absolute error under 2^-39 of the maximum.  sigma_h is clamped to
// [-100, 100] (and 0 for a head without finite nonzero values).
//
// vmax_kernel: per (head, chunk of tokens) the largest |x| as bf16 bits
// (the sign cleared, non-negative bf16 values order like their bit
// patterns); pack_kernel reduces the head's chunks (head_sigma), derives
// sigma_h, and writes it once per head.
static __global__ __launch_bounds__(256) void vmax_kernel(const uint4* __restrict__ v,
                                                   uint32_t* __restrict__ chunk_max, Dims d,
                                                   int nchunk) {
  const int c = wg_x(), h = wg_y(), T = lid_x();
  const int per = (d.n + nchunk - 1) / nchunk;
  const int t0 = c * per, t1 = min(d.n, t0 + per);
  const uint4* src = v + (size_t)h * d.n * 8;
  uint32_t m = 0;
  for (int i = t0 * 8 + T; i < t1 * 8; i += 256) {
    const uint4 x = src[i];
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) m = max(m, max(w[e] & 0x7fffu, (w[e] >> 16) & 0x7fffu));
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  __shared__ uint32_t red[4];
  if ((T & 63) == 0) red[T >> 6] = m;
  __syncthreads();
  if (T == 0) chunk_max[h * kAbsmaxChunks + c] = max(max(red[0], red[1]), max(red[2], red[3]));
}

__global__ __launch_bounds__(256) void pack_kernel(const uint4* __restrict__ k,
                                                   const uint4* __restrict__ v,
                                                   uint4* __restrict__ kp,
                                                   uint4* __restrict__ vt,
                                                   const uint32_t* __restrict__ chunk_max,
                                                   int* __restrict__ vsig, Dims d, int nchunk) {
  __shared__ uint16_t sv[64][66];
  __shared__ int sig_s;
  const int kp0 = wg_x() * 64, h = wg_y(), T = lid_x();
  if (T < 64) {
    const int sig = head_sigma(chunk_max, h, nchunk, T);
    if (T == 0) {
      sig_s = sig;
      if (wg_x() == 0) vsig[h] = sig;
    }
  }
  const size_t src_head = (size_t)h * d.n * 8;
  uint4 vv[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = T + 256 * i;
    const int row = c >> 3, ch = c & 7;
    const int tok = packed_token(kp0 + row, d);
    uint4 kv = make_uint4(0, 0, 0, 0);
    vv[i] = make_uint4(0, 0, 0, 0);
    if (tok >= 0) {
      kv = k[src_head + (size_t)tok * 8 + ch];
      vv[i] = v[src_head + (size_t)tok * 8 + ch];
    }
    kp[((size_t)h * d.ntot_pad + kp0 + row) * 8 + ch] = kv;
  }
  __syncthreads();
  const int sig = sig_s;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = T + 256 * i;
    const int row = c >> 3, ch = c & 7;
    const uint32_t wv[4] = {vv[i].x, vv[i].y, vv[i].z, vv[i].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // bf16 -> float32 (exact) -> times 2^sigma (exact) -> float16 (exact in range)
      const float lo = __builtin_amdgcn_ldexpf(__uint_as_float(wv[e] << 16), sig);
      const float hi = __builtin_amdgcn_ldexpf(__uint_as_float(wv[e] & 0xffff0000u), sig);
      sv[row][ch * 8 + 2 * e] = __builtin_bit_cast(uint16_t, (_Float16)lo);
      sv[row][ch * 8 + 2 * e + 1] = __builtin_bit_cast(uint16_t, (_Float16)hi);
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = T + 256 * i;
    const int dr = c >> 3, kc = c & 7;
    uint32_t wv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      wv[e] = (uint32_t)sv[8 * kc + 2 * e][dr] | ((uint32_t)sv[8 * kc + 2 * e + 1][dr] << 16);
    vt[(((size_t)h * 64 + dr) * d.ntot_pad + kp0) / 8 + kc] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
  }
}

// Packed buffer: K rows, V^T, then the per-head exponent table (H ints) and
// the per-(head, chunk) maxima of vmax_kernel (H x 64 uint32), each region
// 256-byte aligned.
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
static size_t pack_kv_bytes(const Dims& d) {
  return 2 * (size_t)d.H * d.ntot_pad * kHeadDim * sizeof(uint16_t);
}
static int* packed_vsig(const Dims& d, const uint16_t* kp) {
  return (int*)((char*)kp + pack_kv_bytes(d));
}
static uint32_t* packed_chunk_max(const Dims& d, const uint16_t* kp) {
  return (uint32_t*)((char*)kp + pack_kv_bytes(d) + align256((size_t)d.H * sizeof(int)));
}

size_t pack_bytes(const Dims& d) {
  return pack_kv_bytes(d) + align256((size_t)d.H * sizeof(int)) +
         align256((size_t)d.H * kAbsmaxChunks * sizeof(uint32_t));
}

hipError_t launch_absmax(const Dims& d, const uint16_t* x, uint32_t* chunk_max, hipStream_t st) {
  vmax_kernel<<<dim3(absmax_chunks(d), d.H), 256, 0, st>>>((const uint4*)x, chunk_max, d,
                                                         absmax_chunks(d));
  return hipGetLastError();
}

hipError_t launch_pack(const Dims& d, const uint16_t* k, const uint16_t* v, uint16_t* kp,
                       uint16_t* vt, hipStream_t st) {
  const int nchunk = absmax_chunks(d);
  uint32_t* cm = packed_chunk_max(d, kp);
  hipError_t e = launch_absmax(d, v, cm, st);
  if (e != hipSuccess) return e;
  pack_kernel<<<dim3(d.ntot_pad / 64, d.H), 256, 0, st>>>(
      (const uint4*)k, (const uint4*)v, (uint4*)kp, (uint4*)vt, cm, packed_vsig(d, kp), d, nchunk);
  return hipGetLastError();
}

// Workgroup shapes: 128-row blocks run four waves over 128-key tiles (32 KB
// of LDS), 64-row blocks two waves over 64-key tiles; three waves per SIMD.
template <int QT, int KT, int MODE, int WPE = 3>
static hipError_t run_attn(const AttnArgs& a, hipStream_t st) {
  attn_kernel<QT, KT, MODE, WPE><<<xcd_grid(a.n_items), 2 * QT, 0, st>>>(a);
  return hipGetLastError();
}
template <int MODE>
static hipError_t run_attn_b(const Dims& d, const AttnArgs& a, hipStream_t st) {
  return d.b == 64 ? run_attn<64, 64, MODE>(a, st) : run_attn<128, 128, MODE>(a, st);
}

static AttnArgs base_args(const Dims& d, const uint16_t* q, const uint16_t* kp,
                          const uint16_t* vt, uint16_t* o, float* lse) {
  AttnArgs a = {};
  a.q = q;
  a.kp = kp;
  a.vt = vt;
  a.o = o;
  a.lse = lse;
  a.vsig = packed_vsig(d, kp);
  a.d = d;
  return a;
}

hipError_t launch_sparse_attn(const Dims& d, const uint16_t* q, const uint16_t* kp,
                              const uint16_t* vt, const int32_t* row_ptr,
                              const int32_t* col_idx, uint16_t* o, float* lse, hipStream_t st) {
  AttnArgs a = base_args(d, q, kp, vt, o, lse);
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.n_items = d.H * d.B;
  a.patch_only = 1;
  return run_attn_b<kSparseFused>(d, a, st);
}

// kSparseTail plan: slots per XCD (three 128 x 128 workgroups per compute
// unit; 96 when the device cannot be queried) and the compact slot count of the
// pieces of every XCD's last, partial round.
struct TailPlan {
  int m, rows, rows_per_xcd, pieces, slots, grid, max_rem;
};
// Workgroup slots of the current device for 128 x 128 workgroups: three per
// compute unit (768 when the device cannot be queried).
static int device_slots() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      cus >= kXcds / 2)
    return 3 * cus;
  return 768;
}

static TailPlan tail_plan(const Dims& d, int rows_per_head) {
  TailPlan p;
  p.m = device_slots() / kXcds;
  p.rows = d.H * rows_per_head;
  p.rows_per_xcd = (p.rows + kXcds - 1) / kXcds;
  p.pieces = 0;
  p.slots = 0;
  p.grid = 0;
  // Pieces per leftover row.  A largest leftover of at most half a round:
  // as many pieces as let them all run in one round of slots.  A fuller last
  // round: the count p <= kMaxTailPieces whose pieces, in ceil(max_rem p /
  // m) rounds of 1/p of a row each, finish first (plus about one key tile
  // of the row, 1 / (B + 1) of it, per piece for its prologue and partial
  // store), if that beats 0.8 of a row; else the round runs unsplit.
  int max_rem = 0;
  for (int x = 0; x < kXcds; ++x) {
    const int n_x = min(p.rows, (x + 1) * p.rows_per_xcd) - x * p.rows_per_xcd;
    if (n_x > 0) max_rem = max(max_rem, n_x % p.m);
  }
  p.max_rem = max_rem;
  if (max_rem == 0) return p;
  if (p.m / max_rem >= 2) {
    p.pieces = min(kMaxTailPieces, p.m / max_rem);
  } else {
    double best = 0.8;
    for (int pc = 2; pc <= kMaxTailPieces; ++pc) {
      const double cost =
          (double)((max_rem * pc + p.m - 1) / p.m) / pc + (double)pc / (rows_per_head + 1);
      if (cost < best) {
        best = cost;
        p.pieces = pc;
      }
    }
    if (p.pieces == 0) return p;
  }
  for (int x = 0; x < kXcds; ++x) {
    const int n_x = min(p.rows, (x + 1) * p.rows_per_xcd) - x * p.rows_per_xcd;
    if (n_x <= 0) break;
    const int full = n_x / p.m * p.m, rem = n_x - full;
    p.slots = x * (p.rows_per_xcd % p.m) + rem;  // the last non-empty XCD's base + its rows
    p.grid = max(p.grid, full + rem * p.pieces);
  }
  p.slots *= p.pieces;
  return p;
}
static size_t tail_part_o_bytes(const TailPlan& p) {
  return ((size_t)p.slots * 128 * kHeadDim * sizeof(float) + 255) & ~(size_t)255;
}

// Workspace of the patch-row call.  b = 128: the split last round (pieces'
// float32 partials).  b = 64: the aligned-pair lists, then the split last
// round of the pair rows.
static size_t tail_bytes(const TailPlan& p) {
  return tail_part_o_bytes(p) + (size_t)p.slots * 128 * 2 * sizeof(float);
}
static size_t perm_bytes(const Dims& d) {
  return d.B <= 4096 ? (((size_t)d.H * d.B * sizeof(int32_t) + 255) & ~(size_t)255) : 0;
}
size_t patch_rows_workspace(const Dims& d) {
  if (d.b == 128) return tail_bytes(tail_plan(d, d.B)) + perm_bytes(d);
  if (!pairable(d)) return 0;  // the unpaired 64-row kernel needs none
  return pair_cols_bytes(d) + pair_len_bytes(d) + tail_bytes(tail_plan(d, pair_rows(d)));
}

template <bool PAIR, bool O32 = false>
static hipError_t launch_rows_128(const Dims& d, AttnArgs a, int rows_per_head, void* tail_ws,
                                  size_t tail_ws_bytes, hipStream_t st) {
  a.n_items = d.H * rows_per_head;
  const TailPlan p = tail_plan(d, rows_per_head);
  if (!PAIR && tail_ws != nullptr && perm_bytes(d) > 0 &&
      tail_ws_bytes >= tail_bytes(p) + perm_bytes(d)) {
    int32_t* perm = (int32_t*)((char*)tail_ws + tail_bytes(p));
    row_order_kernel<<<dim3((d.B + 255) / 256, d.H), 256, 0, st>>>(a.row_ptr, d, perm);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.row_perm = perm;
  }
  if (tail_ws != nullptr && p.slots > 0 && tail_ws_bytes >= tail_bytes(p)) {
    a.part_o = (float*)tail_ws;
    a.part_ml = (float*)((char*)tail_ws + tail_part_o_bytes(p));
    a.rows_per_xcd = p.rows_per_xcd;
    a.tail_m = p.m;
    a.tail_pieces = p.pieces;
    attn_kernel<128, 128, kSparseTail, 3, PAIR, O32><<<kXcds * p.grid, 256, 0, st>>>(a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    tail_merge_kernel<<<dim3(kXcds * p.max_rem, 128 / 4), 256, 0, st>>>(
        a.part_o, a.part_ml, a.o, a.lse, d, p.rows, p.rows_per_xcd, p.m, p.pieces, p.max_rem,
        rows_per_head, a.row_perm, O32 ? a.o32 : nullptr);
    return hipGetLastError();
  }
  attn_kernel<128, 128, kSparseFused, 3, PAIR, O32><<<xcd_grid(a.n_items), 256, 0, st>>>(a);
  return hipGetLastError();
}

bool patch_rows_train_supported(const Dims& d) { return d.b == 128 || pairable(d); }

// o32 != null (training mode) needs a workspace and b = 128 or aligned pairs
// (b = 64, B <= 8192); the caller checks both.
hipError_t launch_patch_rows(const Dims& d, const uint16_t* q, const uint16_t* kp,
                             const uint16_t* vt, const int32_t* row_ptr, const int32_t* col_idx,
                             uint16_t* o, float* lse, hipStream_t st, void* ws, size_t ws_bytes,
                             float* o32) {
  AttnArgs a = base_args(d, q, kp, vt, o, lse);
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.n_items = d.H * d.B;
  a.o32 = o32;
  if (ws != nullptr && d.b == 128)
    return o32 ? launch_rows_128<false, true>(d, a, d.B, ws, ws_bytes, st)
               : launch_rows_128<false>(d, a, d.B, ws, ws_bytes, st);
  if (ws != nullptr && pairable(d) && ws_bytes >= pair_cols_bytes(d) + pair_len_bytes(d)) {
    int32_t* pc = (int32_t*)ws;
    int32_t* pl = (int32_t*)((char*)ws + pair_cols_bytes(d));
    const hipError_t e = launch_pair_csr(d, row_ptr, col_idx, pc, pl, st);
    if (e != hipSuccess) return e;
    a.pair_cols = pc;
    a.pair_len = pl;
    const size_t used = pair_cols_bytes(d) + pair_len_bytes(d);
    return o32 ? launch_rows_128<true, true>(d, a, pair_rows(d), (char*)ws + used,
                                             ws_bytes - used, st)
               : launch_rows_128<true>(d, a, pair_rows(d), (char*)ws + used, ws_bytes - used, st);
  }
  if (o32 != nullptr) return hipErrorInvalidValue;
  return run_attn_b<kSparseFused>(d, a, st);
}

struct SplitPlan {
  int q_tiles, nsplit, tps;
};
// Key ranges of the special queries: the split count that minimises
// rounds of workgroups x (tiles per workgroup + one tile's worth of prologue
// and partial store), fewest splits on ties (less to reduce).
static SplitPlan special_plan(const Dims& d) {
  SplitPlan p;
  p.q_tiles = d.ns_pad / 128;
  const int nt = d.ntot_pad / 128;
  const long slots = device_slots(), per_split = (long)d.H * p.q_tiles;
  p.tps = nt;
  p.nsplit = 1;
  long best = -1;
  for (int want = 1; want <= min(nt, 1024); ++want) {
    const int tps = (nt + want - 1) / want, ns = (nt + tps - 1) / tps;
    const long cost = (per_split * ns + slots - 1) / slots * (tps + 1);
    if (best < 0 || cost < best) {
      best = cost;
      p.tps = tps;
      p.nsplit = ns;
    }
  }
  return p;
}

size_t special_workspace(const Dims& d) {
  if (d.ns == 0) return 0;
  const SplitPlan p = special_plan(d);
  const size_t slots = (size_t)d.H * d.ns_pad * p.nsplit;
  return ((slots * kHeadDim * sizeof(float) + 255) & ~(size_t)255) + slots * 2 * sizeof(float);
}

hipError_t launch_special_rows(const Dims& d, const uint16_t* q, const uint16_t* kp,
                               const uint16_t* vt, uint16_t* o, float* lse, void* ws,
                               hipStream_t st, float* o32) {
  if (d.ns == 0) return hipSuccess;
  const SplitPlan p = special_plan(d);
  const size_t slots = (size_t)d.H * d.ns_pad * p.nsplit;
  AttnArgs a = base_args(d, q, kp, vt, o, lse);
  a.part_o = (float*)ws;
  a.part_ml = (float*)((char*)ws + ((slots * kHeadDim * sizeof(float) + 255) & ~(size_t)255));
  a.q_tiles = p.q_tiles;
  a.nsplit = p.nsplit;
  a.tiles_per_split = p.tps;
  a.n_items = d.H * p.q_tiles * p.nsplit;
  if (o32 != nullptr)
    attn_kernel<128, 128, kSpecialSplit, 3, false, true><<<xcd_grid(a.n_items), 256, 0, st>>>(a);
  else
    attn_kernel<128, 128, kSpecialSplit, 3><<<xcd_grid(a.n_items), 256, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int items = d.H * d.ns;
  special_reduce_kernel<<<(items + 3) / 4, 256, 0, st>>>(a.part_o, a.part_ml, o, lse, d, p.nsplit,
                                                         o32);
  return hipGetLastError();
}

hipError_t launch_special(const Dims& d, const uint16_t* q, const uint16_t* kp,
                          const uint16_t* vt, uint16_t* o, float* lse, void* ws, hipStream_t st) {
  if (d.ns == 0) return hipSuccess;
  hipError_t e = launch_special_rows(d, q, kp, vt, o, lse, ws, st, nullptr);
  if (e != hipSuccess) return e;
  AttnArgs b = base_args(d, q, kp, vt, o, lse);
  b.q_tiles = d.np_pad / 128;
  b.n_items = d.H * b.q_tiles;
  return run_attn<128, 128, kPatchSpecial>(b, st);
}

hipError_t launch_dense(const Dims& d, const uint16_t* q, const uint16_t* kp, const uint16_t* vt,
                        uint16_t* o, float* lse, hipStream_t st) {
  AttnArgs a = base_args(d, q, kp, vt, o, lse);
  a.q_tiles = d.ntot_pad / 128;
  a.n_items = d.H * a.q_tiles;
  return run_attn<128, 128, kDense>(a, st);
}

}  // namespace bsga
