// The uint4-cache instances of the split-K partial pass with grouped query
// heads (G = 2, 4, 8; attn_split.h).  This unit is compiled with the MFMA
// accumulators kept in VGPRs (-mllvm -amdgpu-mfma-vgpr-form): otherwise the
// P.V accumulators sit in AGPRs and every stage copies them to VGPRs and
// back (about 300 accvgpr moves in the loop).  Measured on MI355X, uint4 K/V
// of 8 rows x 8 KV heads x 32768 tokens: G = 2 / 4 / 8 took 65.5-66 /
// 68.5-70 / 90-92 us against 69-70 / 73-74 / 94-95 us, identical results.
// The one-head instances stay in attn.hip, without the option: they have few
// accumulators, and at the OPT-30B shape the option measured 92.8 and 97.8 us
// against 92.1-92.4.
#include "attn_split.h"

namespace da {
namespace {

template <int QF, int G>
SplitFnPtr pick_u4_one() {
    if constexpr (Cfg<FMT_U4, QF, 128, G>::ok) return attn_split_kernel<FMT_U4, QF, 128, G, false>;
    else return nullptr;
}

template <int QF>
SplitFnPtr pick_u4_g(int G) {
    switch (G) {
    case 2: return pick_u4_one<QF, 2>();
    case 4: return pick_u4_one<QF, 4>();
    case 8: return pick_u4_one<QF, 8>();
    default: return nullptr;
    }
}

}  // namespace

SplitFnPtr pick_split_u4(int qf, int D, int G) {
    if (D != 128) return nullptr;
    if (qf == FMT_F16) return pick_u4_g<FMT_F16>(G);
    if (qf == FMT_F32) return pick_u4_g<FMT_F32>(G);
    return nullptr;
}

}  // namespace da
