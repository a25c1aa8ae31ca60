// Host-side entry points shared between the C-ABI source files of libmuon_rocm.so.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>

#include "../../include/muon_rocm.h"

namespace muon {

// Sets this thread's muon_last_error() text and returns `code`; an empty text clears it.
int set_last_error(int code, const std::string& what);

// rownorm_update on a scratch buffer of scratch_cap bytes that get_scratch returns for
// the current device (NULL with *error set on failure). Validates and plans on the host
// before get_scratch is called; rejects matrices whose RowNorm workspace exceeds
// scratch_cap with MUON_ERR_WORKSPACE. Enqueues no timing events.
int rownorm_noalloc_impl(const muon_matrix* mats, int32_t count, const muon_hparams* hp, float* update_rms,
                         void* stream, size_t scratch_cap, void* (*get_scratch)(std::string* error));

}  // namespace muon
