// Device-side checks shared by the launchers.
#pragma once

#include "fa.h"

namespace fa {

// FA_OK when the current HIP device is a gfx950 (cached per device),
// FA_ERR_UNSUPPORTED for another architecture, FA_ERR_HIP if HIP fails.
fa_status device_check();

}  // namespace fa
