// Paged prefill attention on the matrix cores (MFMA) of gfx950.
//
// Prefill takes all new tokens of a prompt in one pass and is bound by matrix
// products ("vLLM -- PagedAttention으로 ...", section "Prefill vs Decode");
// every new token attends causally -- to itself and to earlier positions only
// ("[Hacker News 요약] ... 'Tiny-vLLM' 직접 구축하기", section "고성능 추론을
// 위한 고급 최적화 기법") -- over K/V read from the paged pool through the
// sequence's block table, GQA as in decode.  Sequence i's n_i new tokens are
// its last n_i context positions: new token j is position L_i - n_i + j, and
// the positions before the new ones are a prefix already in the pool (a cached
// prompt prefix or an earlier chunk).
//
// Tiles: the same 16x16 MFMA tiles as the decode kernel, with the 16 columns
// now (new-token position, q head) pairs: column c of a column group is q head
// kvh*G + c % G of the group's position c / G, so a group covers 16 / G
// positions.  A wave owns CG consecutive column groups and walks the key
// sub-tiles (16 keys) from key 0 up to its last position, each sub-tile used
// by all CG groups:
//
//   S^T[16 keys x 16 cols] = K . Q^T    (D/32 mfma 16x16x32 per group)
//   O^T[D x 16 cols]      += V^T . P^T  (D/16 mfma 16x16x16 per group)
//
// The sub-tiles go in pairs, and P.V takes both at once: D/16 mfma 16x16x32
// over 32 keys per group (on gfx950 one 16x16x32 product keeps the matrix core
// as long as one 16x16x16, so this halves P.V's share).  The four waves of a
// workgroup walk the same keys, so each pair is loaded once per workgroup,
// through LDS: with every wave loading its own (the decode kernel's per-wave
// register ring), the CUs' texture-address units were the bound.
//
// Online softmax per column in fp32 (log2 domain), P rounded to the 16-bit type
// as in decode; the running reference is moved only when a score exceeds it by
// more than a fixed slack, so most sub-tiles need no rescaling of the
// accumulators (the result is the same: softmax does not depend on the
// shift); each lane computes its scores' exponents against the current
// reference and tests their maximum against the slack, and the column maxima
// are folded across lanes only when a test fires.  A key is visible to a
// column when it is not after the column's position; sub-tiles entirely
// before the workgroup's first position need no mask.
// Every wave sees every key its columns need, so nothing is combined across
// waves: each lane divides and stores its columns' outputs itself.
//
// Work items: (sequence, kv head, chunk of NW * CG * 16/G new tokens), the
// chunks of a sequence in descending order so the long causal rows start
// first.  Items past a sequence's new tokens return at once.
#include <type_traits>

#include "decode_mfma_kernel.h"

namespace pkv {

namespace {

// Headroom of the lazily moved softmax reference, log2 units (probabilities up
// to 2^8 before the reference catches up; exact in bf16 and fp16).
constexpr float kRescaleSlack = 8.f;

// Column groups per wave (accumulators of 64 VGPRs at either head_dim) and
// workgroups per CU.  Two workgroups of four waves give each wave 256
// registers.  Measured on the prompt batches: a third workgroup per CU (two or
// three column groups), one workgroup of eight waves, and two pairs per
// barrier were no faster.
template <int D> struct PrefillShape;
template <> struct PrefillShape<64> {
  static constexpr int kGroups = 4, kBlocksPerCu = 2;
};
template <> struct PrefillShape<128> {
  static constexpr int kGroups = 2, kBlocksPerCu = 2;
};

constexpr int kPrefillWaves = 4;

template <typename T, int D, int G, int NW, int CG>
__global__ __launch_bounds__(NW * kWave, PrefillShape<D>::kBlocksPerCu) void prefill_mfma_kernel(PrefillParams p) {
  static_assert(NW * kWave == 256, "shared sub-tiles: whole 16-byte chunks of a step's K and V per thread");
  constexpr int JK = D / 32, JV = D / 16;
  constexpr int QPC = 16 / G;       // positions per column group
  constexpr int QPW = CG * QPC;     // positions per wave

  const int lane = threadIdx.x & (kWave - 1);
  const int r = lane & 15, kg = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

  int it = blockIdx.x;
  const int kvh = it % p.num_kv_heads;
  it /= p.num_kv_heads;
  const int chunk = p.chunks - 1 - it % p.chunks;
  const int seq = it / p.chunks;

  const int s0 = p.query_start[seq];
  const int n = p.query_start[seq + 1] - s0;
  const int first = (chunk * NW + wv) * QPW;  // index of the wave's first new token
  const int first_wg = chunk * NW * QPW;       // the workgroup's
  // every wave of a live workgroup takes part in the loads and barriers; a
  // wave past the last new token computes nothing
  if (s0 < 0 || n <= 0 || s0 + n > p.num_tokens || first_wg >= n) return;
  const bool idle = first >= n;
  const int L = p.context_lens[seq];

  // column (cg, r): new token first + cg*QPC + r/G, q head kvh*G + r%G
  const int head = kvh * G + r % G;
  int idx[CG];
#pragma unroll
  for (int cg = 0; cg < CG; ++cg) idx[cg] = first + cg * QPC + r / G;

  const bool bad_len = L < n || L > p.max_context_len ||
                       static_cast<int64_t>(L) > static_cast<int64_t>(p.max_blocks_per_seq) * p.block_size ||
                       n > p.max_query_len;
  if (bad_len) {
    if (kg == 0) {
#pragma unroll
      for (int cg = 0; cg < CG; ++cg) {
        if (idx[cg] >= n) continue;
        uint16_t* o = p.out + (static_cast<size_t>(s0 + idx[cg]) * p.num_q_heads + head) * D;
        for (int d = 0; d < D; ++d) o[d] = kNanBits<T>;
      }
    }
    return;
  }

  const int p0 = L - n;                          // position of new token 0
  const int last_tok = min(first + QPW, n) - 1;  // the wave's last new token
  const int nsub = idle ? 0 : (p0 + last_tok + 1 + 15) >> 4;
  // sub-tiles the workgroup reads (its last wave's), and those all its waves see whole
  const int nsub_wg = (p0 + min(first_wg + NW * QPW, n) + 15) >> 4;
  const int unmasked_wg = (p0 + first_wg + 1) >> 4;

  // the scale is positive (checked by the caller), so a column's largest
  // score gives its largest exponent
  const float sc2 = p.scale_log2;  // softmax scale * log2(e)
  int pos[CG];
  u32x4 qop[CG][JK];
#pragma unroll
  for (int cg = 0; cg < CG; ++cg) {
    const int t = min(idx[cg], n - 1);  // columns past the last new token repeat it (not stored)
    pos[cg] = p0 + t;
    const uint16_t* qr = p.q + (static_cast<size_t>(s0 + t) * p.num_q_heads + head) * D;
#pragma unroll
    for (int j = 0; j < JK; ++j) qop[cg][j] = *reinterpret_cast<const u32x4*>(qr + (kg + 4 * j) * 8);
  }

  // pool index of sub-tiles win .. win+63, one per lane (-1: a block id outside the pool)
  int tid = 0, win = -1;
  bool bad = false;
  auto fetch_window = [&](int base) {
    const int k = base + lane;
    tid = 0;
    if (k < nsub_wg) {
      const int tok0 = 16 * k;
      const int blk = tok0 / p.block_size;
      const int phys = p.block_tables[static_cast<size_t>(seq) * p.max_blocks_per_seq + blk];
      tid = static_cast<unsigned>(phys) < static_cast<unsigned>(p.num_blocks)
                ? (phys * p.num_kv_heads + kvh) * (p.block_size >> 4) + ((tok0 - blk * p.block_size) >> 4)
                : -1;
    }
    win = base;
  };

  // per column: softmax reference m (log2 units, scale folded in), denominator l
  float m[CG], l[CG];
  f32x4 o[CG][JV];
#pragma unroll
  for (int cg = 0; cg < CG; ++cg) {
    m[cg] = -INFINITY;
    l[cg] = 0.f;
#pragma unroll
    for (int j = 0; j < JV; ++j) o[cg][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // One pair of key sub-tiles (32 keys): q.K per sub-tile, then P.V over both
  // in one 16x16x32 product per 16 dims instead of two 16x16x16 ones.  Lane
  // group kg holds keys 4kg..4kg+3 of the first sub-tile and then 4kg..4kg+3
  // of the second: the order of the keys inside one product is free as long as
  // the V and P operands agree.  Both sub-tiles' scores share one softmax
  // reference.  causal: std::true_type for pairs that some column must not
  // fully see.
  auto compute2 = [&](int q, Tile<D>& ta, Tile<D>& tb, auto causal) {
    const int key0 = 32 * q;
    u32x4 vop[JV];
    {
      u32x2 va[JV], vb[JV];
#pragma unroll
      for (int j = 0; j < JV; ++j) {
        va[j] = v_operand<D>(ta.v, j);
        vb[j] = v_operand<D>(tb.v, j);
      }
      if (decltype(causal)::value && key0 + 32 > L) {
        // keys past the context (the last block's tail) may hold anything: zero
        // their V.  Only a masked pair can reach past the context: every key of
        // an unmasked one precedes the wave's first position
        const int na = L - key0, nb = L - key0 - 16;
        const uint32_t a0 = (4 * kg < na ? 0xffffu : 0u) | (4 * kg + 1 < na ? 0xffff0000u : 0u);
        const uint32_t a1 = (4 * kg + 2 < na ? 0xffffu : 0u) | (4 * kg + 3 < na ? 0xffff0000u : 0u);
        const uint32_t b0 = (4 * kg < nb ? 0xffffu : 0u) | (4 * kg + 1 < nb ? 0xffff0000u : 0u);
        const uint32_t b1 = (4 * kg + 2 < nb ? 0xffffu : 0u) | (4 * kg + 3 < nb ? 0xffff0000u : 0u);
#pragma unroll
        for (int j = 0; j < JV; ++j) {
          va[j].x &= a0;
          va[j].y &= a1;
          vb[j].x &= b0;
          vb[j].y &= b1;
        }
      }
#pragma unroll
      for (int j = 0; j < JV; ++j) vop[j] = u32x4{va[j].x, va[j].y, vb[j].x, vb[j].y};
    }
#pragma unroll
    for (int cg = 0; cg < CG; ++cg) {
      f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < JK; ++j) sa = Mma<T>::qk(ta.k[j], qop[cg][j], sa);
#pragma unroll
      for (int j = 0; j < JK; ++j) sb = Mma<T>::qk(tb.k[j], qop[cg][j], sb);
      const float x[8] = {sa[0], sa[1], sa[2], sa[3], sb[0], sb[1], sb[2], sb[3]};
      bool vis[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        vis[i] = !decltype(causal)::value || key0 + (i >> 2) * 16 + 4 * kg + (i & 3) <= pos[cg];
      // exponents against the current reference, log2 units (masked keys -inf);
      // their maximum needs no quieting of the products' NaNs first, as a
      // maximum of raw scores would
      float y[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = vis[i] ? fmaf(x[i], sc2, -m[cg]) : -INFINITY;
      const float lm = fmaxf(fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3])), fmaxf(fmaxf(y[4], y[5]), fmaxf(y[6], y[7])));
      if (__builtin_amdgcn_ballot_w64(lm > kRescaleSlack)) {
        // the column maxima of the raw scores (the exponents are +inf while
        // the reference is still -inf)
        float xm = -INFINITY;
#pragma unroll
        for (int i = 0; i < 8; ++i) xm = fmaxf(xm, vis[i] ? x[i] : -INFINITY);
        const float bm = max_xor32(max_xor16(xm)) * sc2;
        const bool up = bm > m[cg] + kRescaleSlack;
        const float mn = up ? bm : m[cg];
        const float al = fast_exp2(m[cg] - mn);
        m[cg] = mn;
        l[cg] *= al;
#pragma unroll
        for (int j = 0; j < JV; ++j) o[cg][j] *= al;
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = vis[i] ? fmaf(x[i], sc2, -mn) : -INFINITY;
      }
      uint32_t pw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pw[i] = Mma<T>::pack(fast_exp2(y[2 * i]), fast_exp2(y[2 * i + 1]));
      l[cg] = Mma<T>::sum2(pw[3], Mma<T>::sum2(pw[2], Mma<T>::sum2(pw[1], Mma<T>::sum2(pw[0], l[cg]))));
      const u32x4 pop = {pw[0], pw[1], pw[2], pw[3]};
#pragma unroll
      for (int j = 0; j < JV; ++j) o[cg][j] = Mma<T>::qk(vop[j], pop, o[cg][j]);
    }
  };

  {
    // The workgroup's waves read the same sub-tiles, so each pair is loaded
    // once: its K and V (16 rows of D/8 chunks of 16 bytes each, per
    // sub-tile, contiguous in the pool) come in as 64 * D/8 chunks, D/32 per
    // thread, each load instruction covering one sub-tile's K or V
    // (wave-uniform), two pairs ahead into registers, then stored to one of
    // two LDS slots; every wave reads its K operands and V row slices from
    // LDS.  One workgroup barrier per pair orders the stores of one slot
    // against the reads of the other.  Chunk c of row w sits at chunk
    // c ^ swz(w) of its row, swz taking bits of w that keep the reads of one
    // operand (16 rows, or 16 lanes of one row) and the stores free of bank
    // conflicts (measured: rocprofv3's SQ_LDS_BANK_CONFLICT reads 0 at both
    // head_dims; swz(w) = w at head_dim 128 did not).
    constexpr int CPR = D / 8;                     // chunks per row
    constexpr int CPT = 16 * CPR;                  // chunks of one sub-tile's K (or V)
    constexpr int NL = 4 * CPT / (NW * kWave);     // loads per thread per step
    __shared__ __align__(16) u32x4 kv_lds[2][2][2][CPT];  // [slot][sub-tile][K, V][chunk]
    auto swz = [](int w) { return CPR == 16 ? ((w >> 1) & 7) | ((w & 1) << 3) : (w >> 1) & 7; };
    const int tix = threadIdx.x;
    const int last_wg = nsub_wg - 1;
    const int npair_wg = (nsub_wg + 1) >> 1, upair_wg = unmasked_wg >> 1, npair = (nsub + 1) >> 1;
    // load e of this thread: chunk g = tix + 256 e of the pair, i.e. sub-tile
    // g / (2 CPT), K or V (g / CPT) & 1, chunk u = g % CPT at row u / CPR
    int cst[NL], hsub[NL], hkv[NL], goff[NL];
#pragma unroll
    for (int e = 0; e < NL; ++e) {
      const int g = tix + NW * kWave * e;
      hsub[e] = __builtin_amdgcn_readfirstlane(g / (2 * CPT));
      hkv[e] = __builtin_amdgcn_readfirstlane((g / CPT) & 1);
      const int u = g % CPT, w = u / CPR;
      goff[e] = 16 * u;
      cst[e] = w * CPR + ((u % CPR) ^ swz(w));
    }
    u32x4 stg[2][NL];  // [slot] staging
    auto gload = [&](int q, u32x4 (&a)[NL]) {
      int sub2[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kk = min(2 * q + h, last_wg);
        if ((kk & ~63) != win) fetch_window(kk & ~63);
        int sub = __builtin_amdgcn_readlane(tid, kk & 63);
        bad |= sub < 0 && kk < nsub;  // only the sub-tiles this wave attends to
        sub2[h] = max(sub, 0);
      }
#pragma unroll
      for (int e = 0; e < NL; ++e) {
        const uint16_t* base = (hkv[e] ? p.v_cache : p.k_cache) + static_cast<size_t>(sub2[hsub[e]]) * (16 * D);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0, -1,
                                                                            kBufferConfig);
        a[e] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, goff[e], 0, 0));
      }
    };
    auto lstore = [&](int slot, const u32x4 (&a)[NL]) {
#pragma unroll
      for (int e = 0; e < NL; ++e) kv_lds[slot][hsub[e]][hkv[e]][cst[e]] = a[e];
    };
    auto lread = [&](int slot, int h, Tile<D>& t) {
#pragma unroll
      for (int j = 0; j < JK; ++j) t.k[j] = kv_lds[slot][h][0][r * CPR + ((kg + 4 * j) ^ swz(r))];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int w = 4 * kg + i;
        if constexpr (D == 128) {
          t.v[i].w = kv_lds[slot][h][1][w * CPR + (r ^ swz(w))];
        } else {
          // 8 bytes: half r & 1 of chunk r >> 1
          t.v[i].w = reinterpret_cast<const u32x2*>(&kv_lds[slot][h][1][w * CPR + ((r >> 1) ^ swz(w))])[r & 1];
        }
      }
    };
    // step q: pair q from slot q & 1; the loads of pair q + 2 go out first and
    // pair q + 1 (loaded a step earlier) is stored to the other slot last
    auto step = [&](int q, int slot, auto causal) {
      gload(q + 2, stg[slot]);
      if (q < npair) {
        Tile<D> ta, tb;
        lread(slot, 0, ta);
        lread(slot, 1, tb);
        compute2(q, ta, tb, causal);
      }
      lstore(slot ^ 1, stg[slot ^ 1]);
      __syncthreads();
    };
    gload(0, stg[0]);
    gload(1, stg[1]);
    lstore(0, stg[0]);
    __syncthreads();
    int q = 0;
    // pairs every wave sees whole, then the rest with the causal mask (the
    // loop bounds are the workgroup's, so every wave meets every barrier)
    for (; q + 2 <= upair_wg && q + 2 <= npair_wg; q += 2) {
      step(q, 0, std::false_type{});
      step(q + 1, 1, std::false_type{});
    }
    for (; q < npair_wg; q += 2) {
      step(q, 0, std::true_type{});
      if (q + 1 < npair_wg) step(q + 1, 1, std::true_type{});
    }
  }

  // lane (kg, r) holds rows 4kg+i of O^T for column r: dims (4kg+i)*JV + j
#pragma unroll
  for (int cg = 0; cg < CG; ++cg) {
    float lt = add_xor32(add_xor16(l[cg]));
    if (bad) lt = __int_as_float(0x7fc00000);
    const float inv = 1.f / lt;
    if (idx[cg] >= n) continue;
    uint16_t* orow = p.out + (static_cast<size_t>(s0 + idx[cg]) * p.num_q_heads + head) * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t w[JV / 2];
#pragma unroll
      for (int j = 0; j < JV / 2; ++j)
        w[j] = static_cast<uint32_t>(to_bits<T>(o[cg][2 * j][i] * inv)) |
               (static_cast<uint32_t>(to_bits<T>(o[cg][2 * j + 1][i] * inv)) << 16);
      uint16_t* dst = orow + (4 * kg + i) * JV;
      if constexpr (JV == 4) {
        *reinterpret_cast<u32x2*>(dst) = u32x2{w[0], w[1]};
      } else {
        *reinterpret_cast<u32x4*>(dst) = u32x4{w[0], w[1], w[2], w[3]};
      }
    }
  }
}

template <typename T, int D, int G>
hipError_t launch_t(const PrefillParams& p, hipStream_t stream) {
  constexpr int CG = PrefillShape<D>::kGroups, NW = kPrefillWaves;
  const int per_wg = NW * CG * (16 / G);
  PrefillParams q = p;
  q.chunks = (p.max_query_len + per_wg - 1) / per_wg;
  const int64_t items = static_cast<int64_t>(p.num_seqs) * q.chunks * p.num_kv_heads;
  if (items == 0) return hipSuccess;
  if (items > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_mfma_kernel<T, D, G, NW, CG>),
                     dim3(static_cast<unsigned>(items)), dim3(NW * kWave),
                     0, stream, q);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_g(const PrefillParams& p, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_t<T, D, 1>(p, stream);
    case 2: return launch_t<T, D, 2>(p, stream);
    case 4: return launch_t<T, D, 4>(p, stream);
    case 8: return launch_t<T, D, 8>(p, stream);
    case 16: return launch_t<T, D, 16>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_prefill_mfma(const PrefillParams& p, int dtype, hipStream_t stream) {
  const int group = p.num_q_heads / p.num_kv_heads;
  if (p.head_dim == 64) return dtype == 0 ? launch_g<Bf16, 64>(p, group, stream) : launch_g<Fp16, 64>(p, group, stream);
  return dtype == 0 ? launch_g<Bf16, 128>(p, group, stream) : launch_g<Fp16, 128>(p, group, stream);
}

}  // namespace pkv
