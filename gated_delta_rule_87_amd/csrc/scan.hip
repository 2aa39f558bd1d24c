// State scan + output: per (batch, value head, tile of BV value columns) walk
// the chunks in order, carrying the d_k x BV slice of the state S in MFMA
// accumulators.  Per chunk c (Systolic Linear Attention, Table 2, section 2.3
// and the WY equivalence proof of section 2.4.2):
//
//   Y   = V_c - Kbar_c S_{c-1}                 (C x BV)
//   E_c = diag(beta) A_c Y  = U_c - W_c S_{c-1} (the chunk writes)
//   O_c = Qbar_c S_{c-1} + L_c E_c              (readout; L_c includes t = j)
//   S_c = F_c S_{c-1} + Khat_c^T E_c            (Delta S_c = Khat_c^T E_c)
//
// Every chunk quantity (diag(beta) A_c, L_c, Kbar_c, Qbar_c, Khat_c^T and
// the diagonal of F_c) was prepared by the prep kernel as a ready MFMA
// operand, so this kernel, the only sequential part of the forward pass,
// does no exponentials and forms no operand from the inputs: it streams
// the chunk's tiles and multiplies.  Value columns never mix in the
// recurrence (each column of S evolves on its own), so tiling d_v across
// workgroups is exact.
//
// Operand precision (bf16 inputs): the prepared operands diag(beta) A_c, L_c,
// Kbar, Qbar and Khat are single fp16 (11 significant bits), and so is the
// per-chunk operand copy of the state S (S itself accumulates in fp32
// registers); the intermediates Y and E are kept in LDS as split fp16 pairs
// (x = hi + lo, hi = fp16(x)).  E = diag(beta) A Y and the readout L E use
// both halves (two fp16 MFMAs, fp32 accumulation); the state update
// Khat^T E uses hi alone.  bf16 (8 bits) is too coarse for Qbar, Khat, L,
// S, Y and E: rounding any one of them to bf16 breaks a 1e-2 max-error bar
// on the per-channel-gate workload.  Measured at full size: the single fp16
// E in the state update leaves the error of o where it was and doubles that
// of the final state (at most 4.3e-3, C = 128 stress workload); single fp16
// Y and E everywhere would raise the error of o to 9e-3 there.
//
// Organisation.  Eight waves, two per SIMD, so one wave's memory and LDS
// latency hides behind the other's arithmetic.  Jobs per chunk: Y, E and O
// over (16-token row block, 16-column tile), S over (16-channel block,
// tile).  The state and the intermediate Y and E live in LDS as B operands
// between phases.  The step is bound by the bytes each CU moves through its
// vector memory path, so every tile is fetched once per workgroup, in wide
// pieces: each wave loads only its own Kbar, Qbar and Khat^T rows into
// registers; the nonzero blocks of diag(beta) A_c and L_c, v_c and o_c move
// through LDS as whole-row pieces shared by all threads.  Every operand of chunk
// c+1 (v: c+2) is requested while chunk c computes: Kbar, Qbar and Khat^T
// right after the last use of the registers they go to (they need most of a
// chunk to arrive), the A and L blocks at the end of the E phase, one phase
// after their registers free up (requested together with Kbar and Qbar they
// slow the chunk down).  All loads of a non-final chunk are unconditional
// (indices clamped to the last chunk) so the compiler's memory-wait counts
// stay exact across iterations; the final, possibly ragged chunk is peeled.
//
// Chunk-boundary momentum (kMom; Systolic Linear Attention, Table 2, Z_c,
// mu, kappa_c, and section 2.3): the increment Delta S_c = Khat_c^T E_c goes
// to its own accumulator, the momentum buffer Z (fp32 accumulators shaped
// like S) becomes Z = mu kappa_c Z + Delta S_c, and S = F_c S + Z.  kappa_c is
// 0 when a document starts inside the chunk, which the prep kernels mark by
// writing F_c as -0 (an exponential never yields it).
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace gdr {

constexpr int kScanWaves = 8;
constexpr int kXcds = 8;   // accelerator complex dies of the MI355X, each with its own L2

// FB: bytes of one 16 x 32 operand block in the workspace (fp16 1 KiB, fp32 2 KiB).
// XF: the transfer pass of the segment-parallel scan, which stages no output
// and no L_c blocks.
template <int C, int DK, int BV, int FB, bool XF = false>
struct ScanLayout {
  static constexpr int S_LD = DK + 8;   // S^T rows (elements), 16-byte pad per bf16 plane
  static constexpr int Y_LD = C + 8;    // Y^T, E^T rows
  static constexpr size_t s_bytes = 4 * (size_t)BV * S_LD;
  static constexpr size_t y_bytes = 4 * (size_t)BV * Y_LD;
  // Y split over channel steps (fewer row blocks than waves, d_k >= 128):
  // partial Y and Qbar S products exchanged through [C/16][BV/16][2][64] f32x4
  static constexpr bool kYSplit = (C / 16 == 4) && DK >= 128;
  static constexpr size_t x_bytes = kYSplit ? (size_t)(C / 16) * (BV / 16) * 2 * 64 * 16 : 0;
  // Row-major staging of one chunk's v tile and o tile (C x BV elements of
  // up to 4 bytes, rows padded by 16 bytes).
  static constexpr size_t st_bytes = (size_t)C * (4 * BV + 16);
  // nonzero blocks of diag(beta) A_c, then of L_c, each followed by one zero block
  static constexpr int NZ = tri_blocks(C / 16);
  static constexpr int NREG = XF ? 1 : 2;     // staged lower-triangular operands: A (and L)
  static constexpr size_t al_bytes = NREG * (size_t)(NZ + 1) * FB;
  static constexpr size_t total = s_bytes + 2 * y_bytes + x_bytes + (XF ? 1 : 2) * st_bytes + al_bytes;
};

// The training forward's per-wave staging of the state it saves each chunk
// (after the layout above): a wave's S rows in the state's element type, so
// they leave as 16-byte pieces of whole rows instead of one element per lane
// in the MFMA layout.  Rows padded by 16 bytes.
template <int DK, int BV, int ES>
struct SaveStage {
  static constexpr int NBLK = DK / 16, NT = BV / 16;
  static constexpr int RPW = NBLK >= kScanWaves ? NBLK / kScanWaves : 1;
  static constexpr int WPR = NBLK >= kScanWaves ? 1 : kScanWaves / NBLK;
  static constexpr int TPW = (NT + WPR - 1) / WPR;
  static constexpr int COLS = 16 * TPW;                  // columns of a wave's state tiles
  static constexpr int PITCH = COLS * ES + 16;           // bytes of one staged row
  static constexpr int PIECES = 16 * RPW * COLS * ES / 16;   // 16-byte pieces per wave
  static constexpr size_t bytes = (size_t)kScanWaves * 16 * RPW * PITCH;
};

// One thread's share when all 64 * kScanWaves threads move a row-major C x BV
// tile of E-byte elements between HBM and LDS: NREP pieces of SW bytes, piece
// k of thread t at byte (k * threads + t) * SW of the unpadded tile.  A wave
// then covers whole rows with 8- or 16-byte accesses instead of one element
// per lane in the MFMA layout (four rows of 16 elements per instruction).
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
template <int C, int BV, int E>
struct RowSegs {
  static constexpr int kThreads = 64 * kScanWaves;
  static constexpr int BYTES = C * BV * E / kThreads;
  static constexpr int SW = BYTES < 16 ? BYTES : 16;
  static constexpr int NREP = BYTES / SW;
  static constexpr int ROWB = BV * E;         // bytes of one tile row
  static constexpr int PITCH = ROWB + 16;     // bytes of one staged row
  static_assert(BYTES >= 4 && BYTES % SW == 0 && ROWB % SW == 0, "row pieces");
  using Vec = typename std::conditional<SW == 4, unsigned,
              typename std::conditional<SW == 8, u32x2, u32x4>::type>::type;
  __device__ static int row(int t, int k) { return (k * kThreads + t) * SW / ROWB; }
  __device__ static int colb(int t, int k) { return (k * kThreads + t) * SW % ROWB; }
};

// Distribution of (block, tile) jobs over the eight waves: with at least
// eight blocks a wave owns blocks w, w+8, ... and every tile of each; with
// fewer, NW/NBLK waves share a block and split its tiles.
template <int NBLK, int NT>
struct WaveJobs {
  static constexpr bool kWide = NBLK >= kScanWaves;
  static constexpr int RPW = kWide ? NBLK / kScanWaves : 1;   // blocks per wave
  static constexpr int WPR = kWide ? 1 : kScanWaves / NBLK;   // waves per block
  static constexpr int TPW = (NT + WPR - 1) / WPR;            // tiles per wave and block
  static constexpr bool kAllTiles = NT % WPR == 0;             // every (wave, u) names a tile < NT
  __device__ static int blk(int w, int r) { return kWide ? w + kScanWaves * r : w % NBLK; }
  __device__ static int tile(int w, int u) { return (kWide ? 0 : w / NBLK) + WPR * u; }
};

// base + off elements, with the byte offset formed in 32 bits so the access
// can use a scalar 64-bit base and a 32-bit vector offset.
template <typename T>
__device__ __forceinline__ T *at(T *base, unsigned off) {
  using B = typename std::conditional<std::is_const<T>::value, const char, char>::type;
  return reinterpret_cast<T *>(reinterpret_cast<B *>(base) + off * (unsigned)sizeof(T));
}

// kXfer: the transfer pass of the segment-parallel scan.  Its columns are
// the d_k columns of the segment's transition J (value input 0, initial
// state the identity) followed by the d_v columns of its offset B (the real
// values, initial state 0); it writes [J | B] and no output.
// kSave (training forward): the state entering each chunk, S_{c-1}, is also
// stored to a.states for the backward pass.
// The body takes its workgroup index bx of gx, its segment sgi (ChunkArgs
// seg0 + the launch's segment slot) and whether it is the sequence's last
// segment (it writes hT).
template <typename TIn, typename TOut, class P, int C, int DK, int BV, bool kMom, bool kXfer = false,
          bool kSave = false>
__device__ __forceinline__ void scan_body(const ChunkArgs &a, int bx, int gx, int sgi, bool last_seg) {
  static_assert(!(kMom && kXfer), "momentum doubles the carried state: no transfer pass");
  static_assert(!(kSave && (kMom || kXfer)), "saved states: plain forward only");
  constexpr int FB = P::kF32 ? 2048 : 1024;
  using Lay = ScanLayout<C, DK, BV, FB, kXfer>;
  using IO = TileIO<P>;
  using Plain = typename P::Plain;
  constexpr int NB = C / 16;                  // token row blocks
  constexpr int NT = BV / 16;                 // column tiles
  using J = WaveJobs<NB, NT>;                 // Y / E / O jobs
  using SJ = WaveJobs<DK / 16, NT>;           // S jobs
  constexpr int KSTEPS = DK / 32;             // contraction steps over channels
  constexpr int CSTEPS = C / 32;              // contraction steps over tokens
  // Y jobs: when two waves share a row block (J::WPR = 2) and the rows are
  // long (d_k >= 128), they split its channel steps (each loads half of the
  // block's Kbar / Qbar rows and forms partial products for every column
  // tile) instead of loading the same rows twice; the partials are summed
  // through LDS by the wave that owns the tile.  The chunk step is bound by
  // the issue of its vector memory instructions, so halving them is worth
  // the extra barrier; at d_k = 64 the two waves split the column tiles.
  constexpr int YS = Lay::kYSplit ? 2 : 1;    // waves splitting a row block's channel steps
  static_assert(!Lay::kYSplit || J::WPR == 2, "channel split needs two waves per row block");
  constexpr int YKS = KSTEPS / YS;            // channel steps per wave in Y
  constexpr int YNT = YS == 1 ? J::TPW : NT;  // tiles a wave forms partial products for

  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int T = a.T;
  const int w = wave_id(), l = lane_id();
  const int lr = l & 15, lq = l >> 4;

  // Workgroup -> (column tile, value head, batch).  Workgroups are handed to
  // the eight XCDs round-robin by linear id; renumbering so that each XCD
  // receives a contiguous range of (head, tile) units puts the d_v / BV tiles
  // of one head, which read the same operand tiles, on one XCD and so behind
  // one L2.
  const int NX = (kXfer ? DK + a.d_v : a.d_v) / BV;
  int unit = bx;
  if (gx % kXcds == 0) unit = (bx % kXcds) * (gx / kXcds) + bx / kXcds;
  const int c0 = (unit % NX) * BV, hv = (unit / NX) % a.H_v, b = unit / (NX * a.H_v);
  const bool jcols = kXfer && c0 < DK;        // transfer pass: columns of J (no value input)
  const int vc0 = kXfer ? c0 - DK : c0;       // first value column of the tile
  // Segment of the sequence: chunks [cb, ce).  One segment (the whole
  // sequence) unless the segment-parallel scan split it.
  const int cb = a.seg_len ? min(sgi * a.seg_len, a.N_c) : 0;
  const int ce = a.seg_len ? min(cb + a.seg_len, a.N_c) : a.N_c;
  const int R = a.H_v / a.H_k;
  const int hk = hv / R;
  const int hb = a.beta_per_key_head ? hk : hv;

  StateLds<P> sT;
  OperandLds<P> yT, eT;
  sT.init(smem_raw, BV, Lay::S_LD);
  yT.init(smem_raw + Lay::s_bytes, BV, Lay::Y_LD);
  eT.init(smem_raw + Lay::s_bytes + Lay::y_bytes, BV, Lay::Y_LD);
  f32x4 *xch = reinterpret_cast<f32x4 *>(smem_raw + Lay::s_bytes + 2 * Lay::y_bytes);
  using VS = RowSegs<C, BV, (int)sizeof(TIn)>;
  using OS = RowSegs<C, BV, (int)sizeof(TOut)>;
  unsigned char *vst = smem_raw + Lay::s_bytes + 2 * Lay::y_bytes + Lay::x_bytes;   // v_c, row-major
  unsigned char *ost = vst + Lay::st_bytes;                                           // o_c, row-major
  unsigned char *alA = ost + (kXfer ? 0 : Lay::st_bytes);                             // diag(beta) A_c blocks
  unsigned char *alL = alA + (Lay::NZ + 1) * FB;                                      // L_c blocks
  const int tid = threadIdx.x;
  // LDS block of (I, s): its compacted position, or the zero block
  auto al_slot = [&](int I, int s) { return s <= I / 2 ? tri_index(I, s) : Lay::NZ; };
  const int yh = YS == 1 ? 0 : w / NB;        // this wave's half of the channel steps (YS = 2)

  const TIn *vp = reinterpret_cast<const TIn *>(a.v);
  TOut *op = reinterpret_cast<TOut *>(a.o);
  const int v_row = a.H_v * a.d_v;   // token stride of v, o
  auto row_ok = [&](int c, int t) { return c * C + t < T; };
  auto at_chunk = [&](auto *p, int row, int c) { return p + ((size_t)b * T + (size_t)c * C) * (size_t)row; };
  auto crow = [&](int c, int t) { return (unsigned)min(t, T - 1 - c * C); };   // clamped token row in chunk c
  auto last = [&](int c) { return min(c, ce - 1); };                            // prefetch index, clamped to the segment
  auto tile = [&](int r, int heads, int head, int c) -> const void * { return ws_tile(a, r, heads, head, b, c); };

  // ---------------------------------------------------- prefetch registers
  Plain fkb[J::RPW][YKS];             // Kbar rows of each row block (this wave's channel steps)
  Plain fqb[J::RPW][YKS];             // Qbar rows
  Plain fkh[SJ::RPW][CSTEPS];         // Khat^T rows (channels) of each S block
  float gm[SJ::RPW];                  // exp(Lambda_C) of S row i0 + 4 lq + (lane & 3) of each block
  // this thread's pieces of the v tile: v_{c+1} (staged in LDS during chunk
  // c) and v_{c+2} (requested during chunk c: v comes from HBM, so it is
  // fetched a chunk further ahead than the operand tiles, most of which the
  // other column tiles of the head have already brought into L2)
  typename VS::Vec vseg[VS::NREP], vnext[VS::NREP];

  // The nonzero blocks of diag(beta) A_c and L_c, 2 NZ FB bytes, are loaded
  // by all threads in pieces of AW bytes (piece p at byte AW p of the A
  // blocks followed by the L blocks) during chunk c-1 and staged in LDS in
  // the Y phase of chunk c, where no wave reads either.
  constexpr int AL_BYTES = Lay::NREG * Lay::NZ * FB / (64 * kScanWaves);
  constexpr int AW = AL_BYTES % 16 == 0 ? 16 : AL_BYTES % 8 == 0 ? 8 : 4;
  constexpr int ANREP = AL_BYTES / AW;
  static_assert(AL_BYTES % AW == 0 && FB % AW == 0, "operand block pieces");
  using AVec = typename std::conditional<AW == 4, unsigned,
               typename std::conditional<AW == 8, u32x2, u32x4>::type>::type;
  AVec alseg[ANREP];
  unsigned al_src[ANREP], al_dst[ANREP];   // byte offsets in the chunk's A or L tile / in LDS
  bool al_isl[ANREP];
#pragma unroll
  for (int k = 0; k < ANREP; ++k) {
    const int byte = (k * 64 * kScanWaves + tid) * AW;
    int j = byte / FB;
    const int off = byte % FB;
    al_isl[k] = j >= Lay::NZ;
    if (al_isl[k]) j -= Lay::NZ;
    int I = 0;
#pragma unroll
    for (int i = 1; i < NB; ++i) I = tri_index(i, 0) <= j ? i : I;
    al_src[k] = (I * CSTEPS + (j - tri_index(I, 0))) * FB + off;
    al_dst[k] = (al_isl[k] ? (Lay::NZ + 1) * FB : 0) + j * FB + off;
  }

  auto load_y = [&](int c) __attribute__((always_inline)) {
    const void *tkb = tile(kWsKB, a.H_k, hk, c), *tqb = tile(kWsQB, a.H_k, hk, c);
#pragma unroll
    for (int r = 0; r < J::RPW; ++r) {
      const int I = J::blk(w, r);
#pragma unroll
      for (int s = 0; s < YKS; ++s) {
        fkb[r][s] = IO::get_plain(tkb, I * KSTEPS + yh * YKS + s, l);
        if constexpr (!kXfer) fqb[r][s] = IO::get_plain(tqb, I * KSTEPS + yh * YKS + s, l);
      }
    }
  };
  // v_c: rows clamped to the last token (the tail's extra rows are masked
  // where they are used); staged in LDS by put_v
  auto load_v = [&](typename VS::Vec (&dst)[VS::NREP], int c) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < VS::NREP; ++k) {
      const int t = VS::row(tid, k);
      if (jcols) {
        dst[k] = typename VS::Vec{};
      } else {
        dst[k] = *reinterpret_cast<const typename VS::Vec *>(
            at(at_chunk(vp, v_row, c), crow(c, t) * v_row + hv * a.d_v + vc0 + VS::colb(tid, k) / (int)sizeof(TIn)));
      }
    }
  };
  auto put_v = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < VS::NREP; ++k)
      *reinterpret_cast<typename VS::Vec *>(vst + VS::row(tid, k) * VS::PITCH + VS::colb(tid, k)) = vseg[k];
  };
  auto v_at = [&](int t, int col) -> float {
    return static_cast<float>(*reinterpret_cast<const TIn *>(vst + t * VS::PITCH + col * (int)sizeof(TIn)));
  };
  // o_c from its LDS staging, whole rows per wave
  auto store_o = [&](int c, auto tail_tag) __attribute__((always_inline)) {
    constexpr bool kTail = decltype(tail_tag)::value;
    TOut *o_c = at_chunk(op, v_row, c);
#pragma unroll
    for (int k = 0; k < OS::NREP; ++k) {
      const int t = OS::row(tid, k);
      const auto val = *reinterpret_cast<const typename OS::Vec *>(ost + t * OS::PITCH + OS::colb(tid, k));
      if (!kTail || row_ok(c, t))
        __builtin_nontemporal_store(   // written once, read by no later launch of this pass
            val, reinterpret_cast<typename OS::Vec *>(at(o_c, t * v_row + hv * a.d_v + c0 + OS::colb(tid, k) / (int)sizeof(TOut))));
    }
  };
  auto load_al = [&](int c) __attribute__((always_inline)) {
    const unsigned char *ta = static_cast<const unsigned char *>(tile(kWsA, a.H_beta, hb, c));
    const unsigned char *tl = static_cast<const unsigned char *>(tile(kWsL, a.H_k, hk, c));
#pragma unroll
    for (int k = 0; k < ANREP; ++k)
      alseg[k] = *reinterpret_cast<const AVec *>((al_isl[k] ? tl : ta) + al_src[k]);
  };
  auto put_al = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < ANREP; ++k) *reinterpret_cast<AVec *>(alA + al_dst[k]) = alseg[k];
  };
  auto load_s = [&](int c) __attribute__((always_inline)) {
    const void *tkh = tile(kWsKH, a.H_k, hk, c);
    const float *tgm = static_cast<const float *>(tile(kWsGM, a.H_k, hk, c));
#pragma unroll
    for (int r = 0; r < SJ::RPW; ++r) {
      const int i0 = 16 * SJ::blk(w, r);
#pragma unroll
      for (int s = 0; s < CSTEPS; ++s) fkh[r][s] = IO::get_plain(tkh, SJ::blk(w, r) * CSTEPS + s, l);
      gm[r] = tgm[i0 + 4 * lq + (lr & 3)];
    }
  };

  // ---------------------------------------------------- state and prologue
  f32x4 S[SJ::RPW][SJ::TPW];
  f32x4 Z[SJ::RPW][SJ::TPW];          // momentum buffer (kMom)
  const size_t sbase = ((size_t)b * a.H_v + hv) * DK * a.d_v;
#pragma unroll
  for (int r = 0; r < SJ::RPW; ++r) {
    const int i0 = 16 * SJ::blk(w, r);
#pragma unroll
    for (int u = 0; u < SJ::TPW; ++u) {
      const int n = SJ::tile(w, u);
      if (n >= NT) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + 4 * lq + e, col = c0 + 16 * n + lr;
        if constexpr (kXfer) {
          S[r][u][e] = (jcols && i == col) ? 1.f : 0.f;   // [I | 0]
        } else {
          S[r][u][e] = a.h0 ? a.h0[(size_t)(sgi - a.seg0) * a.h0_seg_stride + sbase + (size_t)i * a.d_v + col] : 0.f;
        }
        if constexpr (kMom) Z[r][u][e] = a.z0 ? a.z0[sbase + (size_t)i * a.d_v + col] : 0.f;
      }
      sT.put4(16 * n + lr, i0 + 4 * lq, S[r][u]);
    }
  }
  // the zero blocks that stand for the blocks above the diagonal
  for (int i = tid; i < FB / 16; i += 64 * kScanWaves) {
    reinterpret_cast<u32x4 *>(alA + Lay::NZ * FB)[i] = u32x4{0u, 0u, 0u, 0u};
    reinterpret_cast<u32x4 *>(alL + Lay::NZ * FB)[i] = u32x4{0u, 0u, 0u, 0u};
  }
  if (ce > cb) {
    load_y(cb);
    load_v(vseg, cb);
    load_v(vnext, last(cb + 1));
    load_al(cb);
    load_s(cb);
    put_v();
  }
  __syncthreads();

  // One chunk.  Every memory instruction of a non-final chunk is
  // unconditional (prefetch indices are clamped to the last chunk); only the
  // final, possibly ragged chunk masks v and guards its output stores.
  auto step = [&](int c, auto tail_tag) __attribute__((always_inline)) {
    constexpr bool kTail = decltype(tail_tag)::value;
    const int c1 = last(c + 1);
    if constexpr (kSave) {
      // S entering chunk c, through the wave's staging rows: lane (lr, lq)
      // holds rows 4 lq .. 4 lq + 3 of column lr of each of its tiles
      using ST = typename std::conditional<P::kF32, float, f16>::type;   // fp16 for bf16 inputs
      using SS = SaveStage<DK, BV, (int)sizeof(ST)>;
      static_assert(SS::RPW == SJ::RPW && SS::TPW == SJ::TPW && SJ::kAllTiles, "save staging follows the S jobs");
      unsigned char *sv = smem_raw + Lay::total + (size_t)w * 16 * SS::RPW * SS::PITCH;
#pragma unroll
      for (int r = 0; r < SJ::RPW; ++r) {
#pragma unroll
        for (int u = 0; u < SJ::TPW; ++u) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            *reinterpret_cast<ST *>(sv + (16 * r + 4 * lq + e) * SS::PITCH + (16 * u + lr) * (int)sizeof(ST)) =
                static_cast<ST>(S[r][u][e]);
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      ST *st = static_cast<ST *>(a.states) + (((size_t)b * a.H_v + hv) * a.N_c + c) * DK * a.d_v;
      constexpr int PPR = SS::COLS * (int)sizeof(ST) / 16;        // pieces per staged row
#pragma unroll
      for (int k = 0; k < (SS::PIECES + 63) / 64; ++k) {
        const int pc = 64 * k + l;
        if (SS::PIECES % 64 == 0 || pc < SS::PIECES) {
          const int row = pc / PPR, cb = (pc % PPR) * 16;           // staged row, byte in it
          const int r = row / 16, j = cb / (int)sizeof(ST);          // block of the wave, staged column
          const int grow = 16 * SJ::blk(w, r) + row % 16;
          const int gcol = c0 + 16 * SJ::tile(w, j / 16) + j % 16;
          const u32x4 v = *reinterpret_cast<const u32x4 *>(sv + row * SS::PITCH + cb);
          __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(st + (size_t)grow * a.d_v + gcol));
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the staging rows' reads before the next chunk's writes
    }

    // ---- Y = V - Kbar S, and Qbar S
    f32x4 accO[J::RPW][J::TPW];
#pragma unroll
    for (int r = 0; r < J::RPW; ++r) {
      const int I = J::blk(w, r);
      f32x4 accY[YNT], accQ[YNT];             // (partial) products per tile
#pragma unroll
      for (int u = 0; u < YNT; ++u) accY[u] = accQ[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < YKS; ++s) {
#pragma unroll
        for (int u = 0; u < YNT; ++u) {
          // channel split: accumulator 0 is this wave's own tile yh
          const int n = YS == 1 ? J::tile(w, u) : (yh + u) % NT;
          if (!(YS == 2 || J::kAllTiles) && n >= NT) continue;
          const auto fs = sT.get(16 * n + lr, 32 * (yh * YKS + s) + 8 * lq);
          mma(accY[u], fkb[r][s], fs);
          if constexpr (!kXfer) mma(accQ[u], fqb[r][s], fs);
        }
      }
      if constexpr (YS == 2 && NT == 2) {
        // hand the partials of the partner's tile (accumulator 1) to it
        f32x4 *give = xch + ((I * NT + 1 - yh) * 2) * 64;
        give[l] = accY[1];
        give[64 + l] = accQ[1];
        __syncthreads();
        const f32x4 *take = xch + ((I * NT + yh) * 2) * 64;
        accY[0] += take[l];
        accQ[0] += take[64 + l];
      } else if constexpr (YS == 2 && NT == 4) {
        // accumulator u holds tile (yh + u) % 4; this wave owns tiles yh and
        // yh + 2 (accumulators 0 and 2) and hands accumulators 1 and 3 to
        // the partner, then keeps its own two in accumulators 0 and 1
#pragma unroll
        for (int u = 1; u < NT; u += 2) {
          f32x4 *give = xch + ((I * NT + (yh + u) % NT) * 2) * 64;
          give[l] = accY[u];
          give[64 + l] = accQ[u];
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < NT; u += 2) {
          const f32x4 *take = xch + ((I * NT + yh + u) * 2) * 64;
          accY[u / 2] = accY[u] + take[l];
          accQ[u / 2] = accQ[u] + take[64 + l];
        }
      } else if constexpr (YS == 2) {
        static_assert(NT == 1, "channel split for 1, 2 or 4 column tiles");
        // one tile: the yh = 1 wave only contributes its partials
        f32x4 *slot = xch + (I * NT * 2) * 64;
        if (yh == 1) {
          slot[l] = accY[0];
          slot[64 + l] = accQ[0];
        }
        __syncthreads();
        if (yh == 0) {
          accY[0] += slot[l];
          accQ[0] += slot[64 + l];
        }
      }
#pragma unroll
      for (int u = 0; u < J::TPW; ++u) {
        const int n = J::tile(w, u);
        accO[r][u] = accQ[u];
        if (!J::kAllTiles && n >= NT) continue;
        f32x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          y[e] = (!kTail || row_ok(c, 16 * I + 4 * lq + e) ? v_at(16 * I + 4 * lq + e, 16 * n + lr) : 0.f) - accY[u][e];
        yT.put4(16 * n + lr, 16 * I + 4 * lq, y);
      }
    }
    put_al();                                   // A_c, L_c: the last readers of A_{c-1}, L_{c-1} were before the previous barrier
    load_y(c1);
#pragma unroll
    for (int k = 0; k < VS::NREP; ++k) vseg[k] = vnext[k];
    load_v(vnext, last(c + 2));
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);          // keep each phase's work (and waits) in its phase

    // ---- E = diag(beta) A Y
#pragma unroll
    for (int r = 0; r < J::RPW; ++r) {
      const int I = J::blk(w, r);
      f32x4 accE[J::TPW];
#pragma unroll
      for (int u = 0; u < J::TPW; ++u) accE[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < CSTEPS; ++s) {        // all steps: blocks above the diagonal read the zero block
        const Plain fa = IO::get_plain(alA, al_slot(I, s), l);
#pragma unroll
        for (int u = 0; u < J::TPW; ++u) {
          const int n = J::tile(w, u);
          if (J::kAllTiles || n < NT) mma(accE[u], fa, yT.get(16 * n + lr, 32 * s + 8 * lq));
        }
      }
#pragma unroll
      for (int u = 0; u < J::TPW; ++u) {
        const int n = J::tile(w, u);
        if (J::kAllTiles || n < NT) eT.put4(16 * n + lr, 16 * I + 4 * lq, accE[u]);
      }
    }
    load_al(c1);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);

    // ---- O = Qbar S + L E (staged in LDS; stored after the chunk's last barrier)
#pragma unroll
    for (int r = 0; r < (kXfer ? 0 : J::RPW); ++r) {
      const int I = J::blk(w, r);
#pragma unroll
      for (int s = 0; s < CSTEPS; ++s) {        // all steps: blocks above the diagonal read the zero block
        const Plain fl = IO::get_plain(alL, al_slot(I, s), l);
#pragma unroll
        for (int u = 0; u < J::TPW; ++u) {
          const int n = J::tile(w, u);
          if (J::kAllTiles || n < NT) mma(accO[r][u], fl, eT.get(16 * n + lr, 32 * s + 8 * lq));
        }
      }
#pragma unroll
      for (int u = 0; u < J::TPW; ++u) {
        const int n = J::tile(w, u);
        if (!J::kAllTiles && n >= NT) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          st(reinterpret_cast<TOut *>(ost + (16 * I + 4 * lq + e) * OS::PITCH) + 16 * n + lr, accO[r][u][e]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- S = F_c S + Khat^T E
#pragma unroll
    for (int r = 0; r < SJ::RPW; ++r) {
      const int i0 = 16 * SJ::blk(w, r);
      // row 4 lq + e of the block: held by lane e of DPP row lq
      const float g[4] = {dpp_row_bcast<0>(gm[r]), dpp_row_bcast<1>(gm[r]), dpp_row_bcast<2>(gm[r]),
                          dpp_row_bcast<3>(gm[r])};
#pragma unroll
      for (int u = 0; u < SJ::TPW; ++u) {
        if (!SJ::kAllTiles && SJ::tile(w, u) >= NT) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) S[r][u][e] *= g[e];
      }
      if constexpr (kMom) {
        // Delta S_c in its own accumulator; Z = mu kappa_c Z + Delta S_c; S += Z
        const float mk = __builtin_signbit(gm[r]) ? 0.f : a.momentum;
        f32x4 D[SJ::TPW];
#pragma unroll
        for (int u = 0; u < SJ::TPW; ++u) D[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < CSTEPS; ++s) {
#pragma unroll
          for (int u = 0; u < SJ::TPW; ++u) {
            const int n = SJ::tile(w, u);
            if (SJ::kAllTiles || n < NT) mma(D[u], fkh[r][s], eT.get_hi(16 * n + lr, 32 * s + 8 * lq));
          }
        }
#pragma unroll
        for (int u = 0; u < SJ::TPW; ++u) {
          if (!SJ::kAllTiles && SJ::tile(w, u) >= NT) continue;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            Z[r][u][e] = mk * Z[r][u][e] + D[u][e];
            S[r][u][e] += Z[r][u][e];
          }
        }
      } else {
#pragma unroll
        for (int s = 0; s < CSTEPS; ++s) {
#pragma unroll
          for (int u = 0; u < SJ::TPW; ++u) {
            const int n = SJ::tile(w, u);
            if (SJ::kAllTiles || n < NT) mma(S[r][u], fkh[r][s], eT.get_hi(16 * n + lr, 32 * s + 8 * lq));
          }
        }
      }
#pragma unroll
      for (int u = 0; u < SJ::TPW; ++u) {
        const int n = SJ::tile(w, u);
        if (SJ::kAllTiles || n < NT) sT.put4(16 * n + lr, i0 + 4 * lq, S[r][u]);
      }
    }
    load_s(c1);
    put_v();                                    // v_{c+1}: the Y phase above was the last reader of v_c
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!kXfer) store_o(c, tail_tag);   // the next O phase rewrites the staging after two barriers
  };
  // The first chunk is peeled so the loop is entered from an iteration with
  // the same memory-instruction order as its own back edge: the compiler's
  // wait counts at the loop head then allow the whole next-chunk prefetch to
  // stay in flight.
  if (ce - cb > 1) {
    step(cb, std::integral_constant<bool, false>());
    for (int c = cb + 1; c + 1 < ce; ++c) step(c, std::integral_constant<bool, false>());
  }
  if (ce > cb) step(ce - 1, std::integral_constant<bool, true>());

  if constexpr (kXfer) {
    // [J | B] of this segment: [B][H_v][d_k][d_k + d_v] per segment
    const int W = DK + a.d_v;
    float *xo = a.xfer + (size_t)(sgi - a.seg0) * ((size_t)a.B * a.H_v * DK * W) + ((size_t)b * a.H_v + hv) * DK * W;
#pragma unroll
    for (int r = 0; r < SJ::RPW; ++r) {
      const int i0 = 16 * SJ::blk(w, r);
#pragma unroll
      for (int u = 0; u < SJ::TPW; ++u) {
        const int n = SJ::tile(w, u);
        if (n >= NT) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) xo[(size_t)(i0 + 4 * lq + e) * W + c0 + 16 * n + lr] = S[r][u][e];
      }
    }
    return;
  }
  if (a.hT && last_seg) {
#pragma unroll
    for (int r = 0; r < SJ::RPW; ++r) {
      const int i0 = 16 * SJ::blk(w, r);
#pragma unroll
      for (int u = 0; u < SJ::TPW; ++u) {
        const int n = SJ::tile(w, u);
        if (n >= NT) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = i0 + 4 * lq + e, col = c0 + 16 * n + lr;
          a.hT[sbase + (size_t)i * a.d_v + col] = S[r][u][e];
        }
      }
    }
  }
  if (kMom && a.zT) {
#pragma unroll
    for (int r = 0; r < SJ::RPW; ++r) {
      const int i0 = 16 * SJ::blk(w, r);
#pragma unroll
      for (int u = 0; u < SJ::TPW; ++u) {
        const int n = SJ::tile(w, u);
        if (n >= NT) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = i0 + 4 * lq + e, col = c0 + 16 * n + lr;
          a.zT[sbase + (size_t)i * a.d_v + col] = Z[r][u][e];
        }
      }
    }
  }
}

template <typename TIn, typename TOut, class P, int C, int DK, int BV, bool kMom, bool kXfer = false,
          bool kSave = false>
__global__ __launch_bounds__(64 * kScanWaves) void scan_kernel(ChunkArgs a) {
  scan_body<TIn, TOut, P, C, DK, BV, kMom, kXfer, kSave>(a, blockIdx.x, gridDim.x, a.seg0 + blockIdx.y,
                                                          blockIdx.y == gridDim.y - 1);
}

// First phase of the segment-parallel scan, one launch: workgroups
// [0, n_scan) scan segment 0 from h0 (32-column tiles; its final state,
// S_in(1), goes to as.hT), the others run the transfer pass of segments
// 1 .. P-2 (BVX-column tiles, n_xfer workgroups per segment).
template <typename TIn, typename TOut, class P, int C, int DK, int BVX>
__global__ __launch_bounds__(64 * kScanWaves) void scan_split_kernel(ChunkArgs as, ChunkArgs ax, int n_scan,
                                                                     int n_xfer) {
  const int g = blockIdx.x;
  if (g < n_scan) {
    scan_body<TIn, TOut, P, C, DK, 32, false>(as, g, n_scan, 0, true);
  } else {
    const int x = g - n_scan;
    scan_body<TIn, TOut, P, C, DK, BVX, false, true>(ax, x % n_xfer, n_xfer, ax.seg0 + x / n_xfer, false);
  }
}

static size_t scan_lds_bytes(int C, int d_k, int BV, int fb) {
#define GDR_CASE(c_, dk_, bv_) \
  if (C == c_ && d_k == dk_ && BV == bv_) \
    return fb == 1024 ? ScanLayout<c_, dk_, bv_, 1024>::total : ScanLayout<c_, dk_, bv_, 2048>::total;
  GDR_CASE(32, 64, 32) GDR_CASE(32, 128, 32) GDR_CASE(32, 256, 32)
  GDR_CASE(64, 64, 16) GDR_CASE(64, 64, 32) GDR_CASE(64, 128, 16) GDR_CASE(64, 128, 32)
  GDR_CASE(64, 256, 16) GDR_CASE(64, 256, 32) GDR_CASE(128, 64, 16) GDR_CASE(128, 64, 32)
  GDR_CASE(128, 128, 16) GDR_CASE(128, 128, 32) GDR_CASE(128, 256, 16) GDR_CASE(128, 256, 32)
#undef GDR_CASE
  return (size_t)1 << 40;
}

// Value-column tile width: 32 when that already gives a workgroup per CU
// (256 of them), else 16 for more parallelism; 0 if the shape is not
// supported.
int scan_choose_bv(int B, int H_v, int C, int d_k, int d_v, bool in_bf16) {
  const int fb = in_bf16 ? 1024 : 2048;
  if (!(C == 32 || C == 64 || C == 128) || !(d_k == 64 || d_k == 128 || d_k == 256) || d_v % 16 != 0) return 0;
  // C = 32: a 16-column tile would give each thread fewer than 4 bytes of a
  // chunk's v rows to move; 32-column tiles only
  if (C == 32) return (d_v % 32 == 0 && scan_lds_bytes(C, d_k, 32, fb) <= 160 * 1024) ? 32 : 0;
  const size_t cap = 160 * 1024;
  const bool fit32 = d_v % 32 == 0 && scan_lds_bytes(C, d_k, 32, fb) <= cap;
  const bool fit16 = scan_lds_bytes(C, d_k, 16, fb) <= cap;
  const long n32 = (long)B * H_v * (d_v / 32);
  if (fit32 && (n32 >= 256 || !fit16)) return 32;
  return fit16 ? 16 : 0;
}

// ------------------------------------------------ segment-parallel scan
// When the (batch, value head, 32-column tile) units cannot fill the GPU
// (fewer than 256), the sequence is cut into P segments of L chunks
// (Systolic Linear Attention, section 3.3: a chunk's state update is an
// affine map S -> J S + B, and maps compose).
//   1. One launch (scan_split_kernel): segment 0 is scanned from h0, writing
//      its output and its final state S_in(1); beside it, segments 1 .. P-2
//      each scan the columns [J | B] of their own map from [I | 0], without
//      output (the transfer pass).
//   2. Combine (seg_combine_kernel): S_in(p+1) = J_p S_in(p) + B_p, p >= 1.
//   3. The ordinary scan of segments 1 .. P-1 at once, segment p from
//      S_in(p), writing o; the last one writes hT.
// P is the largest count for which both scan launches fit one workgroup per
// CU: (P - 1) scan units, and one scan unit plus P - 2 transfer units.
// Momentum doubles the carried state (S and Z), and the training forward
// keeps its per-chunk states, so both keep one segment.
// Transfer-pass workgroups per segment: (d_k + d_v) / 64 column tiles where
// the lean layout fits, else / 32.
static int xfer_units(int B, int H_v, int C, int d_k, int d_v, bool f32) {
  bool k64 = false;
  const int fb = f32 ? 2048 : 1024;
#define GDR_X64(c_, dk_) \
  if (C == c_ && d_k == dk_) \
    k64 = (fb == 1024 ? ScanLayout<c_, dk_, 64, 1024, true>::total : ScanLayout<c_, dk_, 64, 2048, true>::total) <= \
          160 * 1024;
  GDR_X64(32, 64) GDR_X64(32, 128) GDR_X64(32, 256) GDR_X64(64, 64) GDR_X64(64, 128) GDR_X64(64, 256)
  GDR_X64(128, 64) GDR_X64(128, 128) GDR_X64(128, 256)
#undef GDR_X64
  const int w = (k64 && (d_k + d_v) % 64 == 0) ? 64 : 32;
  return B * H_v * ((d_k + d_v) / w);
}

int scan_segments(int B, int H_v, int N_c, int d_v, int C, int d_k, bool f32) {
  if (d_v % 32 != 0) return 1;
  const long units = (long)B * H_v * (d_v / 32);
  if (units >= 256) return 1;
  const long ux = xfer_units(B, H_v, C, d_k, d_v, f32);
  int P = 2;
  while (P < 17 && P + 1 <= N_c / 6 && (long)P * units <= 256 && units + (long)(P - 1) * ux <= 256) ++P;
  return P >= 3 ? P : 1;                      // two segments would run one after the other
}

size_t scan_seg_bytes(int B, int H_v, int N_c, int d_k, int d_v, int C, bool f32) {
  const int P = scan_segments(B, H_v, N_c, d_v, C, d_k, f32);
  if (P < 2) return 0;
  const size_t unit = (size_t)B * H_v * d_k;
  // [J | B] of segments 1 .. P-2, S_in of segments 1 .. P-1
  return 4 * ((size_t)(P - 2) * unit * (d_k + d_v) + (size_t)(P - 1) * unit * d_v);
}

// S_in of segments 2 .. P-1 for one (batch, value head, 32-column tile):
// S_in(p + 1) = J_p S_in(p) + B_p, in fp32, from S_in(1).  The kernel
// is a chain of P - 1 dependent steps, so its time is load latency, not
// arithmetic: 256 threads each own RT = d_k / 32 rows and 4 columns (column
// group t % 8) and read their rows of J_p with 32 loads in flight per slab.
// (One row per thread, 8 d_k threads, reads S from LDS RT times as often and
// measured slower.)
template <int DK>
constexpr int combine_threads() { return 256; }
template <int DK>
__global__ __launch_bounds__(combine_threads<DK>()) void seg_combine_kernel(ChunkArgs a, int P, float *xstate) {
  constexpr int NTH = combine_threads<DK>();
  constexpr int RT = DK * 8 / NTH;            // rows per thread
  constexpr int QW = 32 / RT < DK / 4 ? 32 / RT : DK / 4;   // float4 per row and slab
  constexpr int NSLAB = DK / (4 * QW);
  static_assert(NSLAB >= 1 && NSLAB * 4 * QW == DK, "slabs cover the rows of J");
  __shared__ float4 sh[DK][8];                // S_in(p), [DK][32]
  const int tid = threadIdx.x, tc = tid & 7, tr = tid >> 3;
  const int c0 = blockIdx.x * 32, hv = blockIdx.y, b = blockIdx.z;
  const int W = DK + a.d_v;
  const size_t unit = (size_t)b * a.H_v + hv;
  const size_t slot = (size_t)a.B * a.H_v * DK * a.d_v;           // elements of one segment's states
  float *xs0 = xstate + unit * DK * a.d_v + c0;       // slot 0: S_in(1), from segment 0's scan
  for (int i = tid; i < DK * 8; i += NTH) {
    const int r = i >> 3, q = i & 7;
    sh[r][q] = *reinterpret_cast<const float4 *>(xs0 + (size_t)r * a.d_v + 4 * q);
  }
  __syncthreads();
  for (int p = 1; p + 1 < P; ++p) {                   // [J_p | B_p] in transfer slot p - 1
    const float *xo = a.xfer + (size_t)(p - 1) * a.B * a.H_v * DK * W + unit * DK * W + (size_t)(tr * RT) * W;
    float4 acc[RT];
#pragma unroll
    for (int j = 0; j < RT; ++j) acc[j] = *reinterpret_cast<const float4 *>(xo + (size_t)j * W + DK + c0 + 4 * tc);
#pragma unroll
    for (int sl = 0; sl < NSLAB; ++sl) {
      float4 jr[RT][QW];                      // rows of J_p, columns 4 QW sl ..
#pragma unroll
      for (int j = 0; j < RT; ++j) {
#pragma unroll
        for (int q = 0; q < QW; ++q)
          jr[j][q] = *reinterpret_cast<const float4 *>(xo + (size_t)j * W + 4 * (QW * sl + q));
      }
#pragma unroll
      for (int q = 0; q < QW; ++q) {
        const int k = 4 * (QW * sl + q);
        const float4 s0 = sh[k][tc], s1 = sh[k + 1][tc], s2 = sh[k + 2][tc], s3 = sh[k + 3][tc];
#pragma unroll
        for (int j = 0; j < RT; ++j) {
          const float4 m = jr[j][q];
          acc[j].x += m.x * s0.x + m.y * s1.x + m.z * s2.x + m.w * s3.x;
          acc[j].y += m.x * s0.y + m.y * s1.y + m.z * s2.y + m.w * s3.y;
          acc[j].z += m.x * s0.z + m.y * s1.z + m.z * s2.z + m.w * s3.z;
          acc[j].w += m.x * s0.w + m.y * s1.w + m.z * s2.w + m.w * s3.w;
        }
      }
    }
    __syncthreads();                          // every thread has read S_in(p)
    float *xs = xs0 + (size_t)p * slot;                // S_in(p + 1) in slot p
#pragma unroll
    for (int j = 0; j < RT; ++j) {
      sh[tr * RT + j][tc] = acc[j];
      *reinterpret_cast<float4 *>(xs + (size_t)(tr * RT + j) * a.d_v + 4 * tc) = acc[j];
    }
    __syncthreads();
  }
}

template <typename TIn, typename TOut, class P, int C, int DK, int BV>
static hipError_t launch_scan_t(const ChunkArgs &a, hipStream_t stream, int segments = 1) {
  const size_t lds = ScanLayout<C, DK, BV, P::kF32 ? 2048 : 1024>::total;
  auto kern = a.momentum != 0.f ? scan_kernel<TIn, TOut, P, C, DK, BV, true>
                                : scan_kernel<TIn, TOut, P, C, DK, BV, false>;
  size_t lds_k = lds;
  if (a.states) {                              // training forward: the shapes the backward pass takes
    if constexpr (C == 64 && DK <= 128 && BV == 32) {
      kern = scan_kernel<TIn, TOut, P, C, DK, BV, false, false, true>;
      lds_k += SaveStage<DK, BV, P::kF32 ? 4 : 2>::bytes;
    } else {
      return hipErrorInvalidValue;
    }
  }
  hipError_t e = allow_full_lds(reinterpret_cast<const void *>(kern));
  if (e != hipSuccess) return e;
  dim3 grid((a.d_v / BV) * a.H_v * a.B, segments);
  hipLaunchKernelGGL(kern, grid, dim3(64 * kScanWaves), lds_k, stream, a);
  return hipGetLastError();
}

template <typename TIn, typename TOut, class P, int C, int DK>
static hipError_t launch_segmented(const ChunkArgs &a, hipStream_t s, int segments) {
  constexpr int FB = P::kF32 ? 2048 : 1024;
  const int L = (a.N_c + segments - 1) / segments;
  segments = (a.N_c + L - 1) / L;
  if (segments < 3) return launch_scan_t<TIn, TOut, P, C, DK, 32>(a, s);
  float *seg = reinterpret_cast<float *>(a.ws + a.wl.seg_off);
  const size_t unit = (size_t)a.B * a.H_v * DK;
  float *xstate = seg + (size_t)(segments - 2) * unit * (DK + a.d_v);
  hipError_t e;
  // 1. segment 0 from h0 (final state to S_in(1)) beside the transfer pass of
  //    segments 1 .. P-2 (64-column tiles where the lean layout fits: fewer
  //    workgroups stream the same operands)
  ChunkArgs as = a, ax = a;
  as.seg_len = ax.seg_len = L;
  as.seg0 = 0;
  as.hT = xstate;
  ax.seg0 = 1;
  ax.xfer = seg;
  const int n_scan = (a.d_v / 32) * a.H_v * a.B;
  auto split = [&](auto bvx) -> hipError_t {
    constexpr int BVX = decltype(bvx)::value;
    auto kern = scan_split_kernel<TIn, TOut, P, C, DK, BVX>;
    const size_t l0 = ScanLayout<C, DK, 32, FB>::total, l1 = ScanLayout<C, DK, BVX, FB, true>::total;
    hipError_t err = allow_full_lds(reinterpret_cast<const void *>(kern));
    if (err != hipSuccess) return err;
    const int n_xfer = ((DK + a.d_v) / BVX) * a.H_v * a.B;
    hipLaunchKernelGGL(kern, dim3(n_scan + (segments - 2) * n_xfer), dim3(64 * kScanWaves), l0 > l1 ? l0 : l1, s,
                       as, ax, n_scan, n_xfer);
    return hipGetLastError();
  };
  constexpr bool k64 = ScanLayout<C, DK, 64, FB, true>::total <= 160 * 1024;
  if (k64 && (DK + a.d_v) % 64 == 0) {
    e = split(std::integral_constant<int, k64 ? 64 : 32>());
  } else {
    e = split(std::integral_constant<int, 32>());
  }
  if (e != hipSuccess) return e;
  // 2. S_in(2) .. S_in(P-1)
  hipLaunchKernelGGL(seg_combine_kernel<DK>, dim3(a.d_v / 32, a.H_v, a.B), dim3(combine_threads<DK>()), 0, s, ax,
                     segments, xstate);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // 3. segments 1 .. P-1, segment p from S_in(p) (slot p - 1)
  ChunkArgs ac = a;
  ac.seg_len = L;
  ac.seg0 = 1;
  ac.h0 = xstate;
  ac.h0_seg_stride = unit * a.d_v;
  return launch_scan_t<TIn, TOut, P, C, DK, 32>(ac, s, segments - 1);
}

template <typename TIn, typename TOut, class P, int C, int DK>
static hipError_t launch_scan_bv(const ChunkArgs &a, hipStream_t s) {
  const int segments = (a.momentum != 0.f || a.states)
                           ? 1
                           : scan_segments(a.B, a.H_v, a.N_c, a.d_v, C, DK, P::kF32);
  if (segments > 1 && a.wl.seg_bytes >= scan_seg_bytes(a.B, a.H_v, a.N_c, DK, a.d_v, C, P::kF32) &&
      scan_lds_bytes(C, DK, 32, P::kF32 ? 2048 : 1024) <= 160 * 1024)
    return launch_segmented<TIn, TOut, P, C, DK>(a, s, segments);
  const int bv = a.states ? 32 : scan_choose_bv(a.B, a.H_v, C, DK, a.d_v, sizeof(TIn) == 2);
  if (bv == 32) return launch_scan_t<TIn, TOut, P, C, DK, 32>(a, s);
  if constexpr (C >= 64) {
    if (bv == 16) return launch_scan_t<TIn, TOut, P, C, DK, 16>(a, s);
  }
  return hipErrorInvalidValue;
}

template <typename TIn, typename TOut, class P>
static hipError_t launch_scan_shape(const ChunkArgs &a, hipStream_t s) {
  switch (a.C * 1000 + a.d_k) {
    case 32064: return launch_scan_bv<TIn, TOut, P, 32, 64>(a, s);
    case 32128: return launch_scan_bv<TIn, TOut, P, 32, 128>(a, s);
    case 32256: return launch_scan_bv<TIn, TOut, P, 32, 256>(a, s);
    case 64064: return launch_scan_bv<TIn, TOut, P, 64, 64>(a, s);
    case 64128: return launch_scan_bv<TIn, TOut, P, 64, 128>(a, s);
    case 64256: return launch_scan_bv<TIn, TOut, P, 64, 256>(a, s);
    case 128064: return launch_scan_bv<TIn, TOut, P, 128, 64>(a, s);
    case 128128: return launch_scan_bv<TIn, TOut, P, 128, 128>(a, s);
    case 128256: return launch_scan_bv<TIn, TOut, P, 128, 256>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_scan(const ChunkArgs &a, bool in_bf16, bool out_bf16, hipStream_t stream) {
  if (in_bf16) {
    if (out_bf16) return launch_scan_shape<bf16, bf16, PrecF16>(a, stream);
    return launch_scan_shape<bf16, float, PrecF16>(a, stream);
  }
  if (out_bf16) return launch_scan_shape<float, bf16, PrecF32>(a, stream);
  return launch_scan_shape<float, float, PrecF32>(a, stream);
}

}  // namespace gdr
