// Status strings and build description of the C ABI (include/winattn.h).
#include "../../include/winattn.h"

extern "C" const char* win_strerror(int status) {
    switch (status) {
        case WIN_OK:
            return "ok";
        case WIN_EINVAL:
            return "invalid argument (geometry, size, null or aliased pointer)";
        case WIN_EUNSUPPORTED:
            return "unsupported dtype, head_dim, row size or alignment";
        case WIN_EOVERFLOW:
            return "size or index exceeds the 32-bit index range";
        case WIN_EDEVICE:
            return "HIP runtime error";
        case WIN_ESCRATCH:
            return "the work needs more than the library's static scratch (WIN_TEXT_SCRATCH_BYTES)";
        default:
            return "unknown status";
    }
}

extern "C" const char* win_build_info(void) {
    return "winattn gfx950 | plan: closed-form host + device fill | permute: wave-per-row 16B lanes, "
           "non-temporal | attn_fwd: S^T=KQ^T and O^T=V^TP^T on mfma_f32_32x32x16_bf16, 4 waves x 32 query rows, "
           "64-key tiles, buffer_load lds double buffer, ds_read_b64_tr_b16 for V, base-2 softmax with a row-sum "
           "overflow check (no row max), value-half issue priority, O rows staged through LDS for whole-row stores, "
           "xcd-grouped grid | rope: fused into the "
           "permute | text: [window | text] key tiles, fp32 per-window workspace";
}
