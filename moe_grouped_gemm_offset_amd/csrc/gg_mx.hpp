// gg_mx.hpp -- the block-scaled (MXFP8) main loop of the M-grouped dgrad
// kernels on gfx950: A (M, K) K-major and the expert's B (N, K), K-major or
// N-major, FP8 codes with one E8M0 scale byte per 32 consecutive K values of
// a row (row-major (rows, K/32) scale arrays whatever the codes' major),
// contracted by v_mfma_scale_f32_32x32x64_f8f6f4 with 64 values of K per
// stage and 128 per load unit.
//
// The scales of 8 stages at a time (16 bytes of each of the tile's operand
// rows) are staged in LDS by dword LDS-writing loads, four row-contiguous
// words per 4 lanes, in two alternating buffers: the next group's words
// arrive with the load units of the current group.  A per-lane scale fetch
// per stage would instead send one cache request per row and stage through
// the vector memory path, more requests than the operand data itself.  With
// the fragments of a stage a lane reads the scale word of each of its
// fragment rows; the MFMA shifts it so that the byte of the K block the lane
// feeds sits in byte 0 (a shift right after the read made the wave wait for
// the LDS there, eight times per half: 5% of the MoE dsReLU).
#pragma once
#include "gg_tile.hpp"

namespace gg {

// Scale staging: two buffers, each holding the scale words of a group of 8
// stages (4 load units; 4 words per row: one word covers 128 K values) for
// the tile's A rows (slots 0 .. TM-1) and B rows (slots TM .. TM+TN-1), 16
// bytes per slot, word w at byte 4 w.  (A stage's word of 32 consecutive
// slots is then read with 2-way bank conflicts, 8 such reads per stage and
// wave.)  Group g lives in buffer g & 1.  Group g+1 comes with units 4g+1 ..
// 4g+4, one slice of 128 slots per unit: the last slice lands with the unit
// group g+1 starts in, and the first is issued only after the barrier that
// follows the last read of group g-1.  Past the last group the slices load
// words no stage reads, which keeps the count of loads per unit fixed.
constexpr int kScaleUnits = 4;
template <class C>
struct ScaleLds {
    static constexpr int kSlots = C::TM + C::TN;
    static constexpr int kBuf = kSlots * 16;                           // bytes per buffer
    static constexpr int kBase = 2 * C::kUnit;                         // after the unit buffers
    static constexpr int kSmem = kBase + 2 * kBuf > C::kLds ? kBase + 2 * kBuf : C::kLds;
    static constexpr int kPerUnit = kSlots / kScaleUnits / 16 / C::kWaves;   // loads per wave
    static_assert(C::TM == C::TN && kPerUnit * 16 * C::kWaves * kScaleUnits == kSlots,
                  "scale slices must split evenly over waves and units");
};

// AB: the codes' FP8 format (0 E4M3, 1 E5M2, A and B alike).
// acc[i][j] += the wave's (32 i, 32 j) blocks of deq(A) deq(B)^T over the
// first K values of each row, for the tile whose A rows start at `a` (scales
// `sfa`) and whose B rows start at `b` (scales `sfb`).  Rows are `ld` bytes
// apart (codes) and ld / 32 bytes apart (scales); K and ld are multiples of
// 128 (whole load units, 4-byte scale words), and rows at or past rows_valid
// / cols_valid contribute zero.  With !B_K, B's codes are N-major instead:
// `b` is the tile's first column at K = 0, K rows ldb bytes apart (its
// scales are as for B_K), and cols_valid is a multiple of 16.  smem holds
// ScaleLds<C>::kSmem bytes.
template <class C, int AB = 0, bool B_K = true>
__device__ __forceinline__ void mx_mainloop(char* smem, const char* a, const char* sfa,
                                            const char* b, const char* sfb, int64_t ld, int64_t K,
                                            int rows_valid, int cols_valid, int am0, int bn0,
                                            f32x16 (&acc)[C::MB][C::NB], int64_t ldb = 0) {
    constexpr int TM = C::TM, TN = C::TN, MB = C::MB, NB = C::NB;
    using S = ScaleLds<C>;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int lr = l & 31, lq = l >> 5;
    const int64_t KB = ld / 32;                  // scale bytes per row
    const int nk = (int)(K / 64);                // stages; K % 128 == 0, so nk is even
    // Scale records end with the K/32 bytes of the tile's last valid row, so
    // rows past the tile edge load zeros and no load passes the end of the
    // last row's K range (when ld > K the next bytes may lie past the
    // array).  Words past K inside other rows are loaded but belong to no
    // stage.
    auto scale_records = [&](int valid, int rows) {
        const int v = valid < rows ? valid : rows;
        return (uint32_t)(v > 0 ? (int64_t)(v - 1) * KB + K / 32 : 0);
    };
    const __amdgpu_buffer_rsrc_t rsa = make_rsrc(sfa, scale_records(rows_valid, TM));
    const __amdgpu_buffer_rsrc_t rsb = make_rsrc(sfb, scale_records(cols_valid, TN));
    char* const sbuf = smem + S::kBase;
    const uint32_t sbuf32 = lds_addr(sbuf);
    const int wu = uniform(w);
    // Slice s (0 .. 3) of a group: slots 128 (s & 1) + 16 (kPerUnit w + t) +
    // (l >> 2) of A (s < 2) or B (s >= 2), t < kPerUnit, lane l taking word
    // l & 3 of its slot.
    constexpr int kSliceSlots = TM / 2;
    const uint32_t sc_off = (uint32_t)((16 * S::kPerUnit * w + (l >> 2)) * KB + 4 * (l & 3));
    // load t (0 .. kPerUnit-1) of slice `slice` of scale group grp
    auto scale_load = [&](int grp, int slice, int t) {
        const int half = slice & 1;
        const bool is_a = slice < 2;
        const int slot0 = kSliceSlots * half + 16 * (S::kPerUnit * wu + t);
        const uint32_t lds = sbuf32 + (grp & 1) * S::kBuf + (is_a ? 0 : TM * 16) + slot0 * 16;
        dma4(is_a ? rsa : rsb, lds, sc_off + (uint32_t)((kSliceSlots * half + 16 * t) * KB + 16 * grp));
    };
    using LB = std::conditional_t<B_K, LoadK<C, TN>, LoadMN8<C>>;
    LoadK<C, TM> la;
    LB lb;
    la.init(ld, rows_valid);
    lb.init(B_K ? ld : ldb, cols_valid);
    constexpr int kLA = LoadK<C, TM>::kN, kLB = LB::kN;
    auto issue = [&](uint32_t st, int u, int i) {
        const int64_t kb = (int64_t)u * 128;
        if (i < kLA) {
            la.template issue<false>(st, a + kb, K - kb, i);
        } else if (i < kLA + kLB) {
            if constexpr (B_K)
                lb.template issue<false>(st + TM * kRowBytes, b + kb, K - kb, i - kLA);
            else
                lb.issue(st + TM * kRowBytes, b + kb * ldb, K - kb, i - kLA);
        } else {
            // units 1 .. 4 carry group 1, 5 .. 8 group 2, ...; unit 0
            // carries a slice of group 0 again (identical words)
            const int v = u > 0 ? u - 1 : 0;
            scale_load(u > 0 ? v / kScaleUnits + 1 : 0, v % kScaleUnits, i - kLA - kLB);
        }
    };
    const int lsh = 8 * lq;
    auto read = [&](const char* st, int kt, FragMx8<C>& f, int g) {
        read_mx8<C, B_K>(st, st + TM * kRowBytes, am0, bn0, kt & 1, f, g);
        // this stage's scale word of the group's row, and the shift that
        // brings this lane's K block to byte 0 (applied at the MFMA, so that
        // no wait for the word sits among the reads)
        const char* buf = sbuf + ((kt / 8) & 1) * S::kBuf + 4 * ((kt % 8) >> 1);
        const int sh = lsh + 16 * (kt & 1);
        f.sh = sh;
        if (g < MB)
            f.sa[g] = *reinterpret_cast<const uint32_t*>(buf + (am0 + 32 * g + lr) * 16);
        else
            f.sb[g - MB] = *reinterpret_cast<const uint32_t*>(buf + (TM + bn0 + 32 * (g - MB) + lr) * 16);
    };
    auto mma = [&](const FragMx8<C>& f, int m0_, int m1_) { mma_mx8<C, AB>(f, acc, m0_, m1_); };
    FragMx8<C> frag[2];
    // Group 0 ahead of unit 0: complete whenever unit 0 is.
#pragma unroll
    for (int s4 = 0; s4 < kScaleUnits; s4++)
#pragma unroll
        for (int t = 0; t < S::kPerUnit; t++)
            scale_load(0, s4, t);
    // (N-major B: the early loads' live ranges spill the main loop)
    pipeline<C, kLA + kLB + S::kPerUnit, MB * NB, MB + NB, B_K>(smem, nk, frag, issue, read, mma);
}

}  // namespace gg
