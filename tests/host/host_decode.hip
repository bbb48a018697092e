// Host-side harness of the device block decoder (routed_experts_bit_amd/csrc/rl_decode.h):
// runs the same Strip code on the CPU so that its indexing can be checked against the oracle
// without a GPU.  Test-only.
#include <stdint.h>
#include <string.h>

#include <vector>

#include "rl_decode.h"

using namespace rl;

template <int QT, bool F16, int STRIP>
static void run(const uint8_t* blocks, int64_t nblocks, float* out) {
    std::vector<uint64_t> val(val_entries<QT>());
    for (int i = 0; i < val_entries<QT>(); ++i) val[i] = val_entry<QT, F16>(i);
    uint32_t tern[256];
    for (int i = 0; i < 256; ++i) tern[i] = tern_entry((uint32_t)i);
    const PtrSrc src{blocks};
    for (int64_t b = 0; b < nblocks; ++b) {
        for (int vs = 0; vs < 256; vs += STRIP) {
            StripRaw<QT, STRIP> raw;
            raw.load(src, (uint32_t)(b * Fmt<QT>::BYTES), vs);
            Strip<QT, STRIP> st;
            st.prepare(raw, tern);
            for (int f = 0; f < STRIP / 8; ++f) {
                u32x4 fr = st.frag(f, val.data());
                for (int i = 0; i < 8; ++i) {
                    uint32_t h = (fr[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
                    float v;
                    if (F16) {
                        v = (float)__builtin_bit_cast(_Float16, (uint16_t)h);
                    } else {
                        uint32_t u = h << 16;
                        memcpy(&v, &u, 4);
                    }
                    out[b * 256 + vs + 8 * f + i] = v * st.d;
                }
            }
        }
    }
}

// fp8 e4m3 (OCP, "fn") encoding of a small integer |v| <= 7, and its value.
static uint32_t e4m3_of_int(int v) {
    if (v == 0) return 0u;
    const uint32_t sign = v < 0 ? 0x80u : 0u;
    int a = v < 0 ? -v : v, e = 0;
    while ((a >> (e + 1)) != 0) ++e;              // a = 2^e * (1 + m/8)
    const uint32_t m = (uint32_t)(((a << 3) >> e) & 7);
    return sign | ((uint32_t)(e + 7) << 3) | m;
}
static float e4m3_value(uint32_t b) {
    const int e = (int)((b >> 3) & 15u), m = (int)(b & 7u);
    const float mag = e == 0 ? (float)m / 8.0f / 64.0f : (1.0f + (float)m / 8.0f) * (float)(1 << e) / 128.0f;
    return (b & 0x80u) ? -mag : mag;
}

// fp8 operands of the T1 byte strips of every lane group, mapped back to block positions
// through t1_kmap and scaled by d.
extern "C" int hd_t1f8(const uint8_t* blocks, int64_t nblocks, float* out) {
    // dword reads relative to the dword boundary at or below the first block (the caller pads
    // the buffer by at least 64 bytes)
    const uint8_t* base4 = (const uint8_t*)((uintptr_t)blocks & ~(uintptr_t)3);
    const PtrSrc src4{base4};
    std::vector<uint64_t> tsel(TSEL_ENTRIES);
    for (int i = 0; i < TSEL_ENTRIES; ++i) tsel[i] = tsel_entry(i);
    uint32_t tbl8[8];
    for (int s = 0; s < 8; ++s) tbl8[s] = s == 0 ? 0u : (e4m3_of_int(-s) | (e4m3_of_int(s) << 16));
    const PtrSrc src{blocks};
    for (int64_t b = 0; b < nblocks; ++b) {
        for (int g = 0; g < 4; ++g) {
            T1Lane8 ln;
            ln.init(g);
            // 64-byte window of dwords from the dword boundary at or below the block start
            const uint32_t blk = (uint32_t)(b * Fmt<QT_T1>::BYTES) + (uint32_t)(blocks - base4);
            uint32_t win[16];
            for (int i = 0; i < 16; ++i) win[i] = src4.dw((blk & ~3u) + 4u * (uint32_t)i);
            T1Raw8 raw;
            raw.load_window(win, blk & 3u, g);
            T1Dec8 dec;
            dec.prep(raw, ln, tbl8);
            uint32_t op[16];
            dec.step(0, ln, tsel.data(), op);
            dec.step(1, ln, tsel.data(), op + 8);
            for (int j = 0; j < 64; ++j)
                out[b * 256 + t1_kmap(g, j)] = dec.d * e4m3_value((op[j >> 2] >> (8 * (j & 3))) & 255u);
        }
    }
    return 0;
}

// 16-bit operands of the Q2B strips of the 16-bit MFMA path for every lane group, mapped back to
// block positions through q2_kmap and scaled by d.
extern "C" int hd_q2w(const uint8_t* blocks, int64_t nblocks, int f16, float* out) {
    const uint8_t* base4 = (const uint8_t*)((uintptr_t)blocks & ~(uintptr_t)3);
    const PtrSrc src4{base4};
    std::vector<uint64_t> qsel(QSEL_ENTRIES);
    for (int i = 0; i < QSEL_ENTRIES; ++i) qsel[i] = qsel_entry(i);
    uint64_t q2row[Q2ROW_ENTRIES];
    for (int i = 0; i < Q2ROW_ENTRIES; ++i) q2row[i] = f16 ? q2row_entry<true>(i) : q2row_entry<false>(i);
    for (int64_t b = 0; b < nblocks; ++b) {
        const uint32_t blk = (uint32_t)(b * Fmt<QT_Q2B>::BYTES) + (uint32_t)(blocks - base4);
        uint32_t win[20];  // 80-byte window from the dword boundary at or below the block start
        for (int i = 0; i < 20; ++i) win[i] = src4.dw((blk & ~3u) + 4u * (uint32_t)i);
        for (int g = 0; g < 4; ++g) {
            Q2Raw16 raw;
            raw.load_window(win, blk & 3u, g);
            Q2Dec16 dec;
            dec.prep(raw, q2row);
            for (int h = 0; h < 2; ++h)
                for (int p = 0; p < 2; ++p) {
                    uint32_t op[8];
                    dec.half(h, p, qsel.data(), op);
                    for (int e = 0; e < 16; ++e) {
                        const int j = 2 * p + e / 8, i = e % 8;
                        const uint32_t bits = (op[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                        float v;
                        if (f16) {
                            v = (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
                        } else {
                            const uint32_t u = bits << 16;
                            memcpy(&v, &u, 4);
                        }
                        out[b * 256 + q2_kmap(g, h, j, i)] = dec.d * v;
                    }
                }
        }
    }
    return 0;
}

extern "C" int hd_decode(int qtype, int f16, int strip, const uint8_t* blocks, int64_t nblocks, float* out) {
#define RL_CASE(Q, F, S) \
    if (qtype == Q && f16 == F && strip == S) { run<Q, F, S>(blocks, nblocks, out); return 0; }
    RL_CASE(QT_Q2B, 0, 64) RL_CASE(QT_Q2B, 1, 64) RL_CASE(QT_Q2B, 0, 32) RL_CASE(QT_Q2B, 1, 32)
    RL_CASE(QT_Q2B, 0, 16) RL_CASE(QT_Q2B, 1, 16)
    RL_CASE(QT_T1, 0, 64) RL_CASE(QT_T1, 1, 64) RL_CASE(QT_T1, 0, 32) RL_CASE(QT_T1, 1, 32)
    RL_CASE(QT_T1, 0, 16) RL_CASE(QT_T1, 1, 16)
#undef RL_CASE
    return -1;
}
