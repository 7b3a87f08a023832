// Stand-ins for the device side of the library in the sanitizer build of its
// host code: every launch reports a HIP error, so a call with valid arguments
// runs the whole host path (argument checks, workspace layout, launch
// arguments) and returns ADAFLASH_E_HIP.  No GPU and no HIP runtime.
#include "../../diffusion_drafter_verification_amd/csrc/adaflash_internal.h"

namespace adaflash {
hipError_t launch(const LaunchArgs&) { return hipErrorInvalidValue; }
hipError_t lh_launch(const LhArgs&) { return hipErrorInvalidValue; }
int timing_enable(int cap) { return cap < 0 ? -1 : 0; }
int timing_read(float*, int) { return 0; }
int timing_every(int n) { return n < 1 ? -1 : 0; }
}  // namespace adaflash

extern "C" const char* hipGetErrorString(hipError_t) { return "launch stubbed out (sanitizer build)"; }
