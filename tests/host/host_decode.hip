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

// fp8 step operands of T1 strips with an identity byte table (bytes = digits), mapped back to
// values through the documented byte order pi and the strip's sub-scales.
extern "C" int hd_frag8_t1(const uint8_t* blocks, int64_t nblocks, float* out) {
    uint32_t tern[256];
    for (int i = 0; i < 256; ++i) tern[i] = tern_entry((uint32_t)i);
    const PtrSrc src{blocks};
    for (int64_t b = 0; b < nblocks; ++b) {
        for (int g = 0; g < 4; ++g) {
            StripRaw<QT_T1, 64> raw;
            raw.load(src, (uint32_t)(b * Fmt<QT_T1>::BYTES), 64 * g);
            Strip<QT_T1, 64> st;
            st.prepare(raw, tern);
            for (int h = 0; h < 2; ++h) {
                uint32_t op[8];
                st.frag8(h, 0x03020100u, op);
                const int s = (int)(st.sb[h] >> 8);
                for (int p = 0; p < 32; ++p) {
                    const int digit = (int)((op[p >> 2] >> (8 * (p & 3))) & 255u);
                    const int v = 16 * (p / 16) + 4 * (p % 4) + (p / 4) % 4;
                    out[b * 256 + 64 * g + 32 * h + v] = st.d * (float)(s * (digit - 1));
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
